/*
 * sla_pisa.h - C ABI of the PISA exact-or-approximate attention forward in libsla (gfx950).
 *
 * The operator ("PISA - Piecewise Sparse Attention per Efficient Diffusion Transformers",
 * Italian technical summary, section 2) for one (batch, head), blocks of `block` adjacent
 * tokens (the last one may be short, r_j tokens), logits x = q k^T / sqrt(d):
 *
 *   statistics  per key block j: centroid kbar_j = mean of its keys, value sum vs_j = sum of its
 *               values, first-order matrix H_j = sum_n (k_n - kbar_j)^T v_n [d x d]; per head
 *               Hbar = mean of H_j over all blocks; M_j = ||H_j - Hbar|| (Frobenius).
 *   routing     (covariance-aware top-k) score_ij = qbar_i . kbar_j / sqrt(d) + ln M_j with qbar_i
 *               the mean query of block i (or without ln M_j); HardTop-k per query block, ties
 *               to the lower index, kept indices ascending.  The score is the logarithm of the
 *               first-order error bound e^{s_ij} M_j of approximating block j.
 *   forward     o_t = N_t / D_t with, for query row t of block i with kept set S_i and the rest U_i
 *               and alpha_tj = exp(q_t . kbar_j / sqrt(d)):
 *                 N_t = sum_{j in S_i} sum_n e^{x_tn} v_n + sum_{j in U_i} alpha_tj vs_j
 *                       + (q_t / sqrt(d)) Hbar sum_{j in U_i} alpha_tj
 *                 D_t = sum_{j in S_i} sum_n e^{x_tn} + sum_{j in U_i} r_j alpha_tj.
 *               topk == n_b gives exact softmax attention.
 *
 * Precision: exact terms as in the SLA2 sparse branch (bf16 MFMA, fp32 accumulation, P in
 * bf16); kbar and vs enter the scan as bf16 (fp32 inputs: kbar as bf16 hi + lo), Hbar as bf16;
 * statistics accumulate in fp32 (bf16 inputs: every product exact).
 *
 * Layouts, problem struct, status codes, ownership and error behaviour as in sla.h (Q, K, V
 * [B][H][N][d] of `dtype`; idx [B][H][n_b][topk] int32 ascending; mask [B][H][n_b][n_b] uint8;
 * O [B][H][N][d] float32; every pointer a caller-owned device pointer; nothing is allocated,
 * nothing synchronised).  `topk` of the problem is used by route and forward only.
 *
 * The statistics buffer (sla_pisa_stats_bytes bytes) holds, at the byte offsets returned by
 * sla_pisa_stats_offsets, in this order:
 *   0 kbar_hi [B][H][n_b][d] bf16     1 kbar_lo [B][H][n_b][d] bf16 (kbar = hi + lo)
 *   2 vsum    [B][H][n_b][d] bf16     3 hbar_t  [B][H][d][d] bf16, Hbar transposed ([v][k])
 *   4 hbar    [B][H][d][d] float32 ([k][v])
 *   5 M       [B][H][n_b] float32     6 lnM     [B][H][n_b] float32 (ln 0 = -inf)
 * It is written by sla_pisa_stats and only read by sla_pisa_route and sla_pisa_forward, so one
 * statistics pass serves any number of routings and forwards over the same K and V.
 */
#ifndef SLA_PISA_H
#define SLA_PISA_H

#include "sla.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Size in bytes of the statistics buffer, and of the scratch workspace of sla_pisa_stats and
 * sla_pisa_route (0 when the problem is invalid or unsupported). */
size_t sla_pisa_stats_bytes(const sla_problem* p);
size_t sla_pisa_workspace_bytes(const sla_problem* p);
/* Byte offsets of the seven statistics arrays listed above. */
int sla_pisa_stats_offsets(const sla_problem* p, size_t offsets[7]);

/* Statistics pass (section 2, pre-computation; covariance-aware routing for M_j): reads K and V
 * twice (block statistics and Hbar, then M_j).  stats_bytes / ws_bytes below the sizes above give
 * SLA_ERR_WORKSPACE. */
int sla_pisa_stats(const sla_problem* p, const void* K, const void* V, void* stats,
                   size_t stats_bytes, void* ws, size_t ws_bytes, hipStream_t stream);

/* Covariance-aware top-k (section 2): covariance = 1 ranks by qbar kbar^T / sqrt(d) + ln M_j,
 * 0 by the attention score alone.  idx (required when topk > 0), mask and scores (the
 * [B][H][n_b][n_b] float32 ranked scores) are outputs; mask and scores may be NULL.  Needs the
 * statistics of the same K, V and sla_pisa_workspace_bytes(p) of workspace. */
int sla_pisa_route(const sla_problem* p, const void* Q, const void* stats, size_t stats_bytes,
                   int covariance, int32_t* idx, uint8_t* mask, float* scores, void* ws,
                   size_t ws_bytes, hipStream_t stream);

/* Forward (section 2, core algorithm and fused-kernel outline): writes O.  idx may come from
 * sla_pisa_route or any other router (ascending, in range, topk entries per query block). */
int sla_pisa_forward(const sla_problem* p, const void* Q, const void* K, const void* V,
                     const void* stats, size_t stats_bytes, const int32_t* idx, float* O,
                     hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* SLA_PISA_H */
