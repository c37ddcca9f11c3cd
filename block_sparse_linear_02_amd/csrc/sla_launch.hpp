// sla_launch.hpp - host-side launchers of the gfx950 kernels (internal to libsla).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace sla {

enum { kF32 = 0, kBF16 = 1 };

struct Dims {
  int B, H, N, d, nb, topk, dtype;
};

// Per-(batch, head) branch flags of alpha-driven branch dropping ([BH] uint32).
enum : uint32_t { kDropLinear = 1u, kDropSparse = 2u };
hipError_t launch_branch_flags(const Dims& p, const float* alpha, float tau, uint32_t* flags,
                               hipStream_t stream);

// Router: pool + project (split bf16 outputs [BH][nb][d]) then scores + HardTop-k.
hipError_t launch_route(const Dims& p, const void* Q, const void* K, const float* Wq,
                        const float* Wk, __bf16* q_hi, __bf16* q_lo, __bf16* k_hi,
                        __bf16* k_lo, int32_t* idx, uint8_t* mask, float* probs,
                        hipStream_t stream);
size_t route_lds_bytes(int nb);
// Block means of Q and K without projection, split bf16 [BH][nb][d] (SVOO's initial centroids).
hipError_t launch_pool_means(const Dims& p, const void* Q, const void* K, __bf16* q_hi,
                             __bf16* q_lo, __bf16* k_hi, __bf16* k_lo, hipStream_t stream);
int route_max_blocks();

// Linear-branch states. Per chunk of `chunk_blocks` key blocks: partial H^T [d][d] and partial
// Z [d]; per block z_j [d]; optionally every h_j [d][d] (K-channel major) in fp32 (hj, literal
// mode), or transposed, h_j^T [d][d] (V-channel major), rounded to bf16 (hj_bf, mask-product
// mode) in slices of 64 entries: [BH][d*d/64][nb][64].
int state_chunk_blocks(const Dims& p, bool h_partials = true);
// flags (optional): heads flagged kDropLinear are skipped.
// q (optional; bf16, d = 128, not with hj or flags): the low-bit sparse branch's per-block K
// codes (row-major [BH][N][d]), V codes (transposed per block, [BH][nb][d][64]) and their scales
// [BH][nb], the same bytes as launch_quantize / launch_quantize_v8t, written on the way.
struct StateQuant {
  uint8_t* k8;
  uint8_t* v8t;
  float* sk;
  float* sv;
  int int8;  // 0: OCP e4m3, 1: symmetric int8
};
hipError_t launch_states(const Dims& p, const void* K, const void* V, float* zb, float* h_part,
                         float* z_part, float* hj, __bf16* hj_bf, hipStream_t stream,
                         const uint32_t* flags = nullptr, const StateQuant* q = nullptr);

// Mask-product mode: the complements of the router's index lists as bit rows
// [BH][nb][mask_words(nb)], then T_i^T = sum_{j not in sel(i)} h_j^T for every query block in
// bf16 [BH][nb][d][d] (V-channel major), from the per-block states h_j^T (bf16).
int mask_words(int nb);
hipError_t launch_mask_bits(const Dims& p, const int32_t* idx, uint32_t* bits,
                            hipStream_t stream);
hipError_t launch_tsel(const Dims& p, const __bf16* hj_bf, const uint32_t* bits, __bf16* t_bf,
                       hipStream_t stream, const uint32_t* flags = nullptr);

// Sparse branch with the linear part from the precomputed T_i (bf16) and zeta from z_j, two
// query blocks per workgroup over the union of their kept blocks (n_b <= 2048).
// Per-row outputs of the forward that the backward reads ([BH][N][d] fp32 for Os, Ol; [BH][N]
// for lse2 = log2 sum_n 2^(s_n c) of the sparse branch, +inf without kept keys, and rden =
// 1 / den, 0 where the linear branch is defined as 0).
struct TrainRows {
  float *Os, *Ol, *lse2, *rden;
};
// flags (optional): a kDropLinear head writes alpha O_s only, a kDropSparse head
// (1 - alpha) O_l only.  tr (optional, bf16 with d = 128): also write the TrainRows.
// out_rows (optional, [BH][N]): O row r goes to row out_rows[r] (TrainRows stay in place).
// order (optional, launch_pair_order): workgroup ids in dispatch order.  pairs (optional,
// launch_pair_match): the two query blocks of pair slot p, else 2p and 2p + 1.
hipError_t launch_sparse_pair(const Dims& p, const void* Q, const void* K, const void* V,
                              const int32_t* idx, const float* alpha, const __bf16* t_bf,
                              const float* Z, const float* zb, float* O, hipStream_t stream,
                              const uint32_t* flags = nullptr, const TrainRows* tr = nullptr,
                              const int32_t* out_rows = nullptr, const int32_t* order = nullptr,
                              const int32_t* pairs = nullptr);
// Dispatch order of the pair kernel (each XCD's workgroups by the size of their union of kept
// blocks, largest first) from those sizes (launch_pair_match): pair_order_ints(p) int32 each
// of size and order.
int pair_order_ints(const Dims& p);
// unequal_heads (branch dropping on): the grid shares every head among all 8 XCDs instead of 4;
// launch_pair_match, launch_pair_order and launch_sparse_pair (flags != null) must agree.
hipError_t launch_pair_order(const Dims& p, const int32_t* size, int32_t* order, bool unequal_heads,
                             hipStream_t stream);
// Query blocks paired by the overlap of their kept sets, in windows of 32 (pairs [BH][npair][2]
// int32, second id -1 for a block alone: pair_match_ints(p) int32), the pairs' union sizes per
// workgroup id (what launch_pair_order ranks; size may be null), and the complement bit rows (as
// launch_mask_bits).
int pair_match_ints(const Dims& p);
hipError_t launch_pair_match(const Dims& p, const int32_t* idx, uint32_t* bits, int32_t* pairs,
                             int32_t* size, bool unequal_heads, hipStream_t stream);
// Debug check of idx (validate.hip): *bad = the number of rows with an entry outside [0, n_b)
// or not strictly ascending.
hipError_t launch_validate_idx(const Dims& p, const int32_t* idx, int* bad, hipStream_t stream);
// SoftTop-k training path (soft.hip, and the SOFT forms of the mask GEMM and the pair kernel;
// bf16, d = 128).  Weighted mask GEMM: T_i = sum_j wt[i][j] h_j with wt [BH][nb][pitch] bf16
// (pitch = tsel_weight_pitch(nb), zero past n_b).  Soft sparse branch: every key block j of
// query block i weighted by msoft [BH][nb][nb] (fp32), zeta_i = Z - sum_j M_ij z_j.
int tsel_weight_pitch(int nb);
hipError_t launch_tsel_weighted(const Dims& p, const __bf16* hj_bf, const __bf16* wt, __bf16* t_bf,
                                hipStream_t stream);
hipError_t launch_sparse_soft(const Dims& p, const void* Q, const void* K, const void* V,
                              const float* msoft, const float* alpha, const __bf16* t_bf,
                              const float* Z, const float* zb, float* O, hipStream_t stream,
                              const TrainRows* tr);
// Pooled means (fp32 [BH][nb][d]) and their projections by Wq, Wk (fp32 [BH][nb][d]).
hipError_t launch_soft_pool(const Dims& p, const void* Q, const void* K, const float* Wq,
                            const float* Wk, float* qbar, float* kbar, float* qt, float* kt,
                            hipStream_t stream);
// SoftTop-k per row: scores s = qt kt^T / sqrt(d), M = sigmoid((s - tau) / T) with sum_j M = topk
// (fp32 [BH][nb][nb]) and wt = bf16(1 - M) [BH][nb][tsel_weight_pitch(nb)].
hipError_t launch_soft_topk(const Dims& p, const float* qt, const float* kt, float temp, float* M,
                            __bf16* wt, hipStream_t stream);
// wt = bf16(1 - M), zero-padded to tsel_weight_pitch(nb).
hipError_t launch_soft_weights(const Dims& p, const float* M, __bf16* wt, hipStream_t stream);
// dM of the sparse branch, per (query block, key block) tile in four parts (32 rows x 32 keys
// each): dmsp [BH][nb][nb][4], the sum over each part of 2^(S c - lse2) (dO_s . v - D).
hipError_t launch_soft_dm_sparse(const Dims& p, const void* Q, const void* K, const void* V,
                                 const __bf16* dOs, const float* lse2, const float* Dr, float* dmsp,
                                 hipStream_t stream);
// dM of the linear branch: dmlin [BH][nb][nb] = -(<dA_i, h_j> + dzeta_i . z_j) from the sliced
// bf16 dA_i^T and h_j^T and the fp32 dzeta [BH][nb][d], z [BH][nb][d].
hipError_t launch_soft_dm_linear(const Dims& p, const __bf16* dA_bf, const __bf16* hj_bf,
                                 const float* dzeta, const float* zb, float* dmlin,
                                 hipStream_t stream);
// ds = SoftTop-k backward of dM = dmsp[..][0] + dmsp[..][1] + dmlin ([BH][nb][nb]; zero for
// topk 0 or n_b), optionally writing dM itself.
hipError_t launch_soft_topk_bwd(const Dims& p, const float* M, const float* dmsp, const float* dmlin,
                                float temp, float* ds, float* dM_out, hipStream_t stream);
// Router backward: dqt = ds kt / sqrt(d), dkt = ds^T qt / sqrt(d) per head, then
// dWq = sum qbar^T dqt, dWk = sum kbar^T dkt over every (b, h) and block (fp32 [d][d]).
// (part: router_bwd_part_floats() fp32 of workspace for the chunk partials of dW)
size_t router_bwd_part_floats();
hipError_t launch_router_bwd(const Dims& p, const float* ds, const float* qbar, const float* kbar,
                             const float* qt, const float* kt, float* dqt, float* dkt, float* dWq,
                             float* dWk, float* part, hipStream_t stream);
// Stage 1: dO = bf16(2 (O - O_full) / count) and the loss partials (one per workgroup of
// kLossThreads rows x channels), then the loss (fixed-order sum); the parameter update.
int soft_loss_parts(const Dims& p);
hipError_t launch_soft_loss(const Dims& p, const float* O, const float* O_full, __bf16* dO,
                            float* parts, float* loss, hipStream_t stream);
hipError_t launch_soft_update(const Dims& p, float* Wq, float* Wk, float* alpha, const float* dWq,
                              const float* dWk, const float* dalpha, float lr_w, float lr_a,
                              hipStream_t stream);
// Reduce the chunk partials (fixed order): H^T as bf16 hi/lo [d][d], Z [d]; optionally H [d][d]
// in fp32 (K-channel major, literal mode); Z alone when h_part is null (mask-product mode).
hipError_t launch_state_reduce(const Dims& p, const float* h_part, const float* z_part,
                               __bf16* ht_hi, __bf16* ht_lo, float* Z, float* h_full,
                               hipStream_t stream);

// Sparse branch (+ fused linear removal + combine): writes O.  fused_linear == 0 writes
// alpha * O_s only (literal mode adds the linear branch afterwards).
hipError_t launch_sparse(const Dims& p, const void* Q, const void* K, const void* V,
                         const int32_t* idx, const float* alpha, const __bf16* ht_hi,
                         const __bf16* ht_lo, const float* Z, const float* zb, float* O,
                         int fused_linear, hipStream_t stream);

// Literal linear apply: O += (1 - alpha) * relu(Q)(H - sum_sel h_j) / relu(Q).(Z - sum_sel z_j).
hipError_t launch_linear_literal(const Dims& p, const void* Q, const int32_t* idx,
                                 const float* alpha, const float* h_full, const float* Z,
                                 const float* hj, const float* zb, float* O, hipStream_t stream);

// Low-bit path (int8 = 0: e4m3 codes, 1: int8 codes).
hipError_t launch_quantize(const Dims& p, const void* X, uint8_t* codes, float* scales,
                           hipStream_t stream, int int8 = 0);
// V codes in the per-block transposed layout [BH][nb][d][64] read by the low-bit PV MFMA.
hipError_t launch_quantize_v8t(const Dims& p, const void* X, uint8_t* codes, float* scales,
                               hipStream_t stream, int int8 = 0);
// fp8 sparse branch, mask-product linear mode: two query blocks per workgroup over the union of
// their kept blocks, T_i (bf16) from memory.  pairs (optional, launch_pair_match): the two query
// blocks of pair slot p, else 2p and 2p + 1.  q8 null: each workgroup quantises its own query
// blocks from Q (sq unused), the same codes and scales as launch_quantize.
hipError_t launch_sparse_pair8(const Dims& p, const void* Q, const uint8_t* q8, const uint8_t* k8,
                               const uint8_t* v8, const float* sq, const float* sk,
                               const float* sv, const int32_t* idx, const float* alpha,
                               const __bf16* t_bf, const float* Z, const float* zb, float* O,
                               hipStream_t stream, int int8 = 0, const int32_t* pairs = nullptr);
hipError_t launch_sparse_fp8(const Dims& p, const void* Q, const void* K, const void* V,
                             const uint8_t* q8, const uint8_t* k8, const uint8_t* v8,
                             const float* sq, const float* sk, const float* sv,
                             const int32_t* idx, const float* alpha, const __bf16* ht_hi,
                             const __bf16* ht_lo, const float* Z, const float* zb, float* O,
                             hipStream_t stream);

// PISA.  Statistics: kbar_j as bf16 hi + lo and vs_j as bf16 ([BH][nb][d] each), Hbar^T in
// bf16 [BH][d][d] ([c][c'], V channel major), Hbar in fp32 [BH][d][d] ([c'][c]), M_j and ln M_j
// in fp32 [BH][nb]; h_part holds the chunk partials ([BH][chunks][d][d], state_chunk_blocks).
hipError_t launch_pisa_stats(const Dims& p, const void* K, const void* V, __bf16* kbar_hi,
                             __bf16* kbar_lo, __bf16* vsum, float* h_part, __bf16* hbar_t,
                             float* hbar, float* M, float* lnM, hipStream_t stream);
// Routing: pooled Q (no projection; split bf16 [BH][nb][d] in q_hi, q_lo) against the centroids,
// plus bias[j] (ln M_j, or null for the attention score alone); scores gets the raw selection
// scores when non-null.
hipError_t launch_pisa_route(const Dims& p, const void* Q, __bf16* q_hi, __bf16* q_lo,
                             const __bf16* kbar_hi, const __bf16* kbar_lo, const float* bias,
                             int32_t* idx, uint8_t* mask, float* scores, hipStream_t stream);
// Forward (n_b <= pisa_max_blocks()).
int pisa_max_blocks();
hipError_t launch_pisa(const Dims& p, const void* Q, const void* K, const void* V,
                       const int32_t* idx, const __bf16* kbar_hi, const __bf16* kbar_lo,
                       const __bf16* vsum, const __bf16* hbar_t, float* O, hipStream_t stream);

// Backward (bwd.hip; bf16, d = 128).  prep: dalpha, dO_s = alpha dO and G = (1 - alpha) dO / den
// in bf16 [BH][N][d], D = dO_s . O_s and e = -G . O_l [BH][N], dzeta_i [BH][nb][d].
hipError_t launch_bwd_prep(const Dims& p, const void* Q, const void* dO, const float* alpha,
                           const TrainRows& tr, float* dalpha, __bf16* dOs, float* Dr, __bf16* G,
                           float* e, float* dzeta, hipStream_t stream);
// The kept sets transposed: bit rows [BH][nb][mask_words(nb)] of the query blocks keeping each
// key block, and the complement within n_b.
hipError_t launch_bits_t(const Dims& p, const int32_t* idx, uint32_t* kept_t, uint32_t* unsel_t,
                         hipStream_t stream);
hipError_t launch_bwd_dz(const Dims& p, const float* dzeta, const uint32_t* kept_t, float* tot,
                         float* dz, hipStream_t stream);
hipError_t launch_bwd_dq(const Dims& p, const void* Q, const void* K, const void* V,
                         const int32_t* idx, const __bf16* dOs, const float* lse2, const float* Dr,
                         const __bf16* G, const float* e, const __bf16* t_bf, const float* Z,
                         const float* zb, float* dQ, hipStream_t stream);
hipError_t launch_bwd_dkv(const Dims& p, const void* Q, const void* K, const void* V,
                          const uint32_t* kept_t, const __bf16* dOs, const float* lse2,
                          const float* Dr, const __bf16* dh, const float* dz, float* dK, float* dV,
                          hipStream_t stream);

// SVOO co-clustering (bf16, d = 128, C = nb clusters).  assign: nearest centroid (split bf16
// [BH][C][d]) of every row of X by inner product -> [BH][N].  order: the stable sort of the
// tokens by cluster -> perm [BH][N] (position -> token) and start [BH][C + 1], through the
// per-segment counts hist [BH][svoo_segments(N)][C].  centroids: member means (empty clusters
// untouched).  permute_rows: y[p] = x[perm[p]] (scatter = 0) or y[perm[p]] = x[p] (scatter = 1)
// for rows of row_bytes (a multiple of 4) of every (batch, head).
int svoo_segments(int N);
hipError_t launch_svoo_assign(const Dims& p, const void* X, const __bf16* c_hi,
                              const __bf16* c_lo, int32_t* assign, hipStream_t stream);
hipError_t launch_svoo_order(const Dims& p, const int32_t* assign, int32_t* hist, int32_t* start,
                             int32_t* perm, hipStream_t stream);
hipError_t launch_svoo_centroids(const Dims& p, const void* X, const int32_t* perm,
                                 const int32_t* start, __bf16* c_hi, __bf16* c_lo,
                                 hipStream_t stream);
hipError_t launch_permute_rows(const Dims& p, const void* X, int row_bytes, const int32_t* perm,
                               void* Y, int scatter, hipStream_t stream);

}  // namespace sla
