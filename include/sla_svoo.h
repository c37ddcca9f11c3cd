/*
 * sla_svoo.h - C ABI of SVOO's online bidirectional co-clustering in libsla (gfx950), and the
 * row permutations that run the SLA2 path on co-clustered blocks.
 *
 * The operation ("Training-Free Sparse Attention for Fast Video Generation via Offline
 * Layer-Wise Sparsity Profiling and Online Bidirectional Co-Clustering", Italian summary,
 * section 2.B) for one (batch, head) with C = n_b clusters:
 *
 *   start       query centroids qc_c and key centroids kc_c = the means of block c of Q and of
 *               K in the original order (blocks of `block` tokens, the last may be short);
 *   iteration   (repeated `iters` times)
 *                 key step    a_k(n) = argmax_c K_n . qc_c, then kc_c = mean of the keys with
 *                             a_k = c;
 *                 query step  a_q(t) = argmax_c Q_t . kc_c, then qc_c = mean of the queries with
 *                             a_q = c;
 *               among equal affinities the lower cluster index wins; a cluster that receives no
 *               member keeps its previous centroid;
 *   order       perm_q = the stable sort of the tokens by a_q (position -> token: clusters in
 *               index order, original order within a cluster), perm_k likewise by a_k.
 *
 * The SLA2 path then runs unchanged on the permuted sequence: Q and alpha gathered by perm_q, K
 * and V by perm_k (sla_svoo_gather), route and forward on the gathered tensors, and the output
 * rows scattered back to the original query order by perm_q (sla_svoo_scatter).  The clusters
 * stay valid over several diffusion steps, so one sla_svoo_cluster call serves many forwards.
 *
 * Precision: affinities by bf16 MFMA on the exact bf16 tokens against centroids split into a
 * bf16 high and low part, fp32 accumulation (about fp32 accuracy); member sums in fp64, the
 * mean rounded to fp32.  Results are deterministic (no floating-point atomics).
 *
 * Layouts, problem struct, status codes, ownership and error behaviour as in sla.h; every
 * pointer is a caller-owned device pointer, nothing is allocated, nothing synchronised.
 * Supported: bf16 Q and K with d = 128 (other dtypes and d give SLA_ERR_UNSUPPORTED).
 */
#ifndef SLA_SVOO_H
#define SLA_SVOO_H

#include "sla.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Scratch workspace of sla_svoo_cluster in bytes (0 when the problem is invalid or
 * unsupported). */
size_t sla_svoo_workspace_bytes(const sla_problem* p);

/* Co-clustering (section 2.B): Q, K [B][H][N][d] bf16; iters in [1, 64].  Writes perm_q, perm_k
 * [B][H][N] int32 (position -> token) and, when not NULL, the clusters q_assign, k_assign
 * [B][H][N] int32 in [0, n_b).  SLA_ERR_INVALID for a NULL input or permutation or iters out of
 * range, SLA_ERR_WORKSPACE for ws_bytes below sla_svoo_workspace_bytes(p). */
int sla_svoo_cluster(const sla_problem* p, const void* Q, const void* K, int32_t iters,
                     int32_t* q_assign, int32_t* k_assign, int32_t* perm_q, int32_t* perm_k,
                     void* ws, size_t ws_bytes, hipStream_t stream);

/* Row permutations of [B][H][N] rows of row_bytes bytes each (a multiple of 4, at most 4096):
 * gather Y[b][h][p] = X[b][h][perm[b][h][p]], scatter Y[b][h][perm[b][h][p]] = X[b][h][p].
 * perm must be a permutation of 0 .. N-1 for every (b, h) (entries are clamped to that range,
 * so a malformed one gives wrong rows but no access outside X and Y); X and Y must not overlap.
 * Q, K, V (d bf16 values a row), alpha (one float) and O (d floats) all fit.  Only p->B, p->H
 * and p->N are read. */
int sla_svoo_gather(const sla_problem* p, const void* X, int32_t row_bytes, const int32_t* perm,
                    void* Y, hipStream_t stream);
int sla_svoo_scatter(const sla_problem* p, const void* X, int32_t row_bytes, const int32_t* perm,
                     void* Y, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* SLA_SVOO_H */
