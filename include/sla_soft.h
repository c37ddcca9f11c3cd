/*
 * sla_soft.h - C ABI of the SoftTop-k training path of SLA2 on MI355X (gfx950).
 *
 * SLA2: Sparse-Linear Attention with Learnable Routing and QAT, Italian summary section 2.B and
 * Arabic summary section 2.ba: while training, the router builds its mask with a differentiable
 * SoftTop-k so that gradients reach proj_q and proj_k (inference uses HardTop-k, sla_route);
 * Arabic summary section 2.dal: stage 1 fits the router and the mixing vector alpha with an MSE
 * loss against full-attention outputs.
 *
 * Reading (the pages do not define SoftTop-k): with the router scores
 * s_ij = (mean(Q_i) proj_q) . (mean(K_j) proj_k) / sqrt(d) (as in sla_route), the soft mask is
 *   M_ij = sigmoid((s_ij - tau_i) / T),   tau_i such that sum_j M_ij = topk,
 * (topk = 0 gives M = 0, topk = n_b gives M = 1), whose limit as the temperature T goes to 0 is
 * the HardTop-k mask.  M weighs the keys of block j in the sparse branch of query block i and
 * 1 - M weighs them in its linear branch:
 *   O_s(q) = sum_n M_{i,b(n)} e^{q.k_n/sqrt(d)} v_n / sum_n M_{i,b(n)} e^{q.k_n/sqrt(d)},
 *   O_l(q) = relu(q) sum_j (1 - M_ij) h_j / relu(q) . sum_j (1 - M_ij) z_j,
 *   O = alpha O_s + (1 - alpha) O_l,
 * with h_j = relu(K_j)^T V_j, z_j = relu(K_j)^T 1; a 0/1 M gives exactly the forward of
 * sla_forward.  Gradients with respect to M follow the chain rule; through SoftTop-k by implicit
 * differentiation of the row budget: ds_ij = (M_ij (1 - M_ij) / T) (dM_ij - sum_l dM_il
 * M_il (1 - M_il) / sum_l M_il (1 - M_il)).
 *
 * Layouts and ownership as in sla.h: Q, K, V [B][H][N][d] bf16 (d = 128 only; other shapes give
 * SLA_ERR_UNSUPPORTED), proj_q / proj_k [d][d] fp32 (y = x W), alpha [B][H][N] fp32,
 * M [B][H][n_b][n_b] fp32, O [B][H][N][d] fp32, dO [B][H][N][d] bf16.  Every pointer is a
 * caller-owned device pointer; the workspace is sla_soft_workspace_bytes(p) bytes.  Arguments
 * are checked on the host before anything is enqueued (null pointers, temperature not a
 * positive finite number: SLA_ERR_INVALID; a short workspace: SLA_ERR_WORKSPACE; a failed
 * launch: SLA_ERR_HIP).  Sums run in a fixed order (no atomics), so results are deterministic.
 */
#ifndef SLA_SOFT_H
#define SLA_SOFT_H

#include "sla.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Workspace of every entry point below (0 when the problem is invalid or unsupported). */
size_t sla_soft_workspace_bytes(const sla_problem* p);

/* SoftTop-k router: M (output) for the budget p->topk at temperature T (> 0). */
int sla_soft_route(const sla_problem* p, const void* Q, const void* K, const float* proj_q,
                   const float* proj_k, float temperature, float* M, void* ws, size_t ws_bytes,
                   hipStream_t stream);

/* Soft-mask forward: O (output) = alpha O_s + (1 - alpha) O_l with the weights M. */
int sla_soft_forward(const sla_problem* p, const void* Q, const void* K, const void* V,
                     const float* M, const float* alpha, float* O, void* ws, size_t ws_bytes,
                     hipStream_t stream);

/* Gradients of <dO, O> for the forward with M = SoftTop-k(proj_q, proj_k, temperature, topk)
 * (M must be sla_soft_route's output for the same arguments): dproj_q, dproj_k [d][d] (summed
 * over every batch and head), dalpha [B][H][N], and optionally dM [B][H][n_b][n_b] (NULL to
 * skip) and the recomputed O (NULL to skip), all overwritten.  Q, K and V are inputs of the fit,
 * not trained here (sla_backward gives their gradients for the hard forward). */
int sla_soft_backward(const sla_problem* p, const void* Q, const void* K, const void* V,
                      const float* proj_q, const float* proj_k, float temperature, const float* M,
                      const float* alpha, const void* dO, float* dproj_q, float* dproj_k,
                      float* dalpha, float* dM, float* O, void* ws, size_t ws_bytes,
                      hipStream_t stream);

/* One stage-1 step: M = SoftTop-k, O = the soft-mask forward, loss = mean((O - O_full)^2)
 * (written to *loss, a device float, before the update), dO = 2 (O - O_full) / count, the
 * gradients, then in place proj_q -= lr_proj dproj_q, proj_k -= lr_proj dproj_k,
 * alpha = clamp(alpha - lr_alpha dalpha, 0, 1).  O_full [B][H][N][d] fp32 is the full-attention
 * output (e.g. sla_forward with every block kept and alpha = 1). */
int sla_stage1_step(const sla_problem* p, const void* Q, const void* K, const void* V,
                    const float* O_full, float* proj_q, float* proj_k, float* alpha,
                    float temperature, float lr_proj, float lr_alpha, float* loss, void* ws,
                    size_t ws_bytes, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* SLA_SOFT_H */
