/*
 * sla.h - C ABI of the MI355X (gfx950) SLA2 hybrid sparse-linear attention inference forward.
 *
 * The operator (SLA2: Sparse-Linear Attention with Learnable Routing and QAT; Italian summary
 * sections 1 and 2, Arabic summary sections 1 and 2) for one (batch, head):
 *
 *   router   Q and K are mean-pooled over blocks of `block` adjacent tokens, projected by the
 *            learnable proj_q / proj_k (y = x @ W), scored s_ij = q~_i . k~_j / sqrt(d), and a
 *            HardTop-k per query block keeps `topk` key blocks (mask M, index list idx).
 *   sparse   O_s: exact softmax attention of each query over the tokens of its kept blocks.
 *   linear   O_l: ReLU-feature linear attention (the kernel function of "SALAD: Achieve
 *            High-Sparsity Attention via Efficient Linear Attention Tuning for Video Diffusion
 *            Transformer", section 2) over the tokens of the unselected blocks,
 *            O_l(q) = relu(q) A_i / (relu(q) . zeta_i), A_i = sum_{j unselected} relu(K_j)^T V_j,
 *            zeta_i = sum_{j unselected} relu(K_j)^T 1; 0 when nothing is unselected or the
 *            denominator is 0.
 *   combine  O = alpha * O_s + (1 - alpha) * O_l  (SLA2 Italian summary section 2.A).
 *   fp8      The sparse branch may run on e4m3-quantised Q, K, P, V (SLA2 Italian summary
 *            section 2.C, Arabic summary section 2.jim); router and linear branch stay
 *            unquantised.
 *
 * Layouts (all row-major, innermost index last, densely packed):
 *   Q, K, V  [B][H][N][d], dtype `dtype` (SLA_BF16 or SLA_F32)
 *   proj_q, proj_k  [d][d] float32, y[c] = sum_r x[r] * W[r][c]; one matrix for every (b, h)
 *   alpha    [B][H][N] float32, mixing weight of the sparse branch per query token
 *   idx      [B][H][n_b][topk] int32, kept key blocks per query block, strictly ascending
 *   mask     [B][H][n_b][n_b] uint8 (1 = kept)
 *   scores   [B][H][n_b][n_b] float32, row softmax of the block-score map
 *   O        [B][H][N][d] float32
 * with n_b = ceil(N / block); the last block may be short (its mean runs over its valid
 * tokens, its missing keys are masked, nothing is stored past N).
 *
 * Ownership: every pointer is a device pointer owned by the caller, including the workspace;
 * the library allocates no device memory, keeps no pointer after a call returns and does not
 * synchronise the host.  Work is enqueued on `stream` in call order; calls are re-entrant.
 *
 * Errors: arguments are checked on the host before anything is enqueued.  A null required
 * pointer, a non-positive size, topk outside [0, n_b] or an element count over 2^62 gives
 * SLA_ERR_INVALID; a shape outside the compiled set (block != 64, d not in {64, 128}, dtype
 * not in sla_dtype) gives SLA_ERR_UNSUPPORTED; a workspace smaller than the matching
 * *_workspace_bytes() gives SLA_ERR_WORKSPACE; a failed launch gives SLA_ERR_HIP (the hipError_t
 * is available from sla_last_hip_error()).  idx contents are trusted (ascending, in range)
 * unless SLA_VALIDATE=1 (sla_validate_idx); non-finite inputs give undefined output.
 */
#ifndef SLA_H
#define SLA_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  SLA_OK = 0,
  SLA_ERR_INVALID = -1,
  SLA_ERR_UNSUPPORTED = -2,
  SLA_ERR_WORKSPACE = -3,
  SLA_ERR_HIP = -4
} sla_status;

typedef enum { SLA_F32 = 0, SLA_BF16 = 1 } sla_dtype; /* dtype of Q, K, V */

typedef struct {
  int32_t B, H, N, d; /* batch, heads, tokens, head dim */
  int32_t block;      /* tokens per block (compiled: 64) */
  int32_t topk;       /* kept key blocks per query block, 0 <= topk <= n_b */
  int32_t dtype;      /* sla_dtype */
} sla_problem;

/* How the forward removes the kept blocks' states from the linear branch.
 * SLA_LINEAR_FUSED (default): the sparse kernel rebuilds sum_sel relu(K_j)^T V_j and
 *   sum_sel relu(K_j)^T 1 on chip from the K/V tiles it already stages for the sparse branch,
 *   subtracts them from the totals H and Z, and applies relu(Q_i) (no per-block d x d state is
 *   stored or read).
 * SLA_LINEAR_LITERAL: every h_j = relu(K_j)^T V_j is materialised in the workspace and a
 *   separate kernel sums the kept ones per query block before applying relu(Q).
 * SLA_LINEAR_MASK_PRODUCT: every h_j is materialised in bf16 and
 *   T_i = sum_{j not in sel(i)} h_j is formed for all query blocks at once as the product of the
 *   complement (unselected) 0/1 mask, built from idx as a bit mask, with the stacked states (one
 *   MFMA GEMM per head, fp32 accumulation), stored in bf16; the sparse kernel applies relu(Q)
 *   to its T_i.  The sparse kernel runs two query blocks per workgroup, paired among nearby
 *   blocks by the overlap of their kept sets; the pairing decides only which blocks share a
 *   workgroup (and its staged K/V tiles): each block still walks its own kept tiles in
 *   ascending order, so its result does not depend on its partner.  The unselected blocks are summed directly, never as H minus the kept ones, so
 *   no cancellation appears when almost every block is kept.  The two bf16 roundings put a relative error
 *   of about 2^-9 on the linear branch's numerator (the other modes keep it near fp32). */
enum { SLA_LINEAR_FUSED = 0, SLA_LINEAR_LITERAL = 1, SLA_LINEAR_MASK_PRODUCT = 2 };

typedef struct {
  int32_t linear_mode;     /* SLA_LINEAR_FUSED, SLA_LINEAR_LITERAL or SLA_LINEAR_MASK_PRODUCT */
  hipEvent_t sparse_begin; /* if non-null: recorded on `stream` right before the sparse kernel */
  hipEvent_t sparse_end;   /* if non-null: recorded on `stream` right after it */
  hipEvent_t states_begin; /* if non-null: recorded right before the linear-state kernels */
  hipEvent_t states_end;   /* if non-null: recorded right after them (state build + reduction) */
  /* Branch dropping ("SALAD: Achieve High-Sparsity Attention via Efficient Linear Attention
   * Tuning for Video Diffusion Transformer", section 2, Post-Tuning Branch Dropping): when
   * branch_drop is non-zero, a (b, h) whose linear weight max_t (1 - alpha_t) is <= drop_tau
   * skips its linear branch (states, mask GEMM, apply) and one whose sparse weight max_t alpha_t
   * is <= drop_tau skips its sparse branch; the dropped term is omitted, the other keeps its
   * weight.  The decision is taken on the GPU from alpha (no host synchronisation).
   * drop_tau = 0 drops only branches whose weight is exactly 0 everywhere (the output is then
   * unchanged).  0 <= drop_tau < 0.5, else SLA_ERR_INVALID; only the bf16 forward in the
   * mask-product linear mode supports it (else SLA_ERR_UNSUPPORTED). */
  int32_t branch_drop;
  float drop_tau;
  /* if non-null: `stream` waits for this event after the linear-state kernels and before the
   * first kernel that reads idx, so that the router (sla_route on another stream, the event
   * recorded after it) overlaps the state build.  The caller keeps idx unchanged until this
   * forward has finished. */
  hipEvent_t idx_ready;
  /* if non-null ([B][H][N] int32, a permutation of 0 .. N-1 per (b, h)): output row r of (b, h)
   * is written to row out_rows[b][h][r] of O, e.g. SVOO's query permutation to return rows of a
   * co-clustered sequence to their original order without a separate scatter.  Entries are
   * clamped to 0 .. N-1 (a malformed permutation misplaces rows, it never writes outside O).
   * Only the bf16 forward in the mask-product mode supports it (else SLA_ERR_UNSUPPORTED). */
  const int32_t* out_rows;
} sla_forward_opts;

/* Workspace sizes in bytes for a problem (0 when the problem is invalid or unsupported). */
size_t sla_route_workspace_bytes(const sla_problem* p);
/* variant: 0 = sla_forward (fused linear), 1 = sla_forward_fp8 (fused linear), 2 = literal
 * linear mode, 3 = mask-product linear mode, 4 = sla_forward_fp8 in the mask-product mode,
 * 5 = sla_forward_int8 (mask-product mode). */
size_t sla_forward_workspace_bytes(const sla_problem* p, int variant);

/* Router (SLA2 Italian summary section 2.B, Arabic summary section 2.ba and 2.dal): block
 * mean-pool of Q and K, projection, block-score map, HardTop-k.  Among equal scores the lower
 * block index is kept; the kept indices are written in ascending order.  mask and scores are
 * optional outputs (NULL to skip).  Needs sla_route_workspace_bytes(p) bytes of workspace. */
int sla_route(const sla_problem* p, const void* Q, const void* K, const float* proj_q,
              const float* proj_k, int32_t* idx, uint8_t* mask, float* scores, void* ws,
              size_t ws_bytes, hipStream_t stream);

/* Forward with the bf16 (or fp32-input) sparse branch: O = alpha O_s + (1 - alpha) O_l
 * (SLA2 Italian summary section 2.A).  topk == 0 gives O_s = 0; topk == n_b gives O_l = 0.
 * Needs sla_forward_workspace_bytes(p, 0) bytes of workspace. */
int sla_forward(const sla_problem* p, const void* Q, const void* K, const void* V,
                const int32_t* idx, const float* alpha, float* O, void* ws, size_t ws_bytes,
                hipStream_t stream);

/* sla_forward with options (linear mode, timing events); opts may be NULL.  Needs
 * sla_forward_workspace_bytes(p, 2) bytes in literal mode, (p, 3) in the mask-product mode,
 * (p, 0) in the fused one. */
int sla_forward_ex(const sla_problem* p, const void* Q, const void* K, const void* V,
                   const int32_t* idx, const float* alpha, float* O, void* ws, size_t ws_bytes,
                   hipStream_t stream, const sla_forward_opts* opts);

/* Forward with the quantised sparse branch (SLA2 Italian summary section 2.C, Arabic summary
 * section 2.jim): Q, K, V are quantised per (b, h, 64-token block) to OCP e4m3 with an absmax
 * scale (x * fp32(448 / absmax), round to nearest even, saturating), P is quantised per
 * (query block x key block) tile with scale max(tile) / 448 over exp(S - rowmax) using the
 * exact row maximum, and O_s = sum (P8 sP)(V8 sV) / sum exp(S - rowmax).  Only dtype
 * SLA_BF16 with d = 128 is compiled.  Needs sla_forward_workspace_bytes(p, 1) bytes.
 * The codes of K and V come out of the linear branch's state kernel, which reads K and V anyway,
 * and in the mask-product mode each workgroup of the sparse kernel quantises its own two query
 * blocks (in the fused mode Q has a launch of its own); with SLA_SEPARATE_QUANT=1 in the
 * environment (read on every call; a debug switch for comparing the two) all three are made by
 * launches of their own.  The bytes, and so the output, are the same either way.  The same
 * holds for sla_forward_int8. */
int sla_forward_fp8(const sla_problem* p, const void* Q, const void* K, const void* V,
                    const int32_t* idx, const float* alpha, float* O, void* ws, size_t ws_bytes,
                    hipStream_t stream);

/* sla_forward_fp8 with options: opts->linear_mode fused (workspace variant 1) or mask product
 * (variant 4: two query blocks per workgroup over the union of their kept blocks, T_i from the
 * mask GEMM); literal is rejected (SLA_ERR_INVALID). */
int sla_forward_fp8_ex(const sla_problem* p, const void* Q, const void* K, const void* V,
                       const int32_t* idx, const float* alpha, float* O, void* ws,
                       size_t ws_bytes, hipStream_t stream, const sla_forward_opts* opts);

/* Forward with the INT8 sparse branch (SLA2 Italian summary section 2.C and Arabic summary
 * section 2.jim name INT8 beside FP8): as sla_forward_fp8 in the mask-product mode with int8
 * codes instead of e4m3: per (b, h, 64-token block) symmetric absmax scales a / 127,
 * code = round-half-even(x * fp32(127 / a)) in [-127, 127]; P per (query block x key block)
 * tile with scale max(tile) / 127 over exp(S - rowmax) (exact row maximum), codes in
 * [0, 127]; S and P V from exact int32 products (v_mfma_i32_32x32x32_i8) times the scales;
 * the denominator sums the unquantised exp(S - rowmax).  Only dtype SLA_BF16 with d = 128 is
 * compiled.  Needs sla_forward_workspace_bytes(p, 5) bytes.  The _ex form takes opts whose
 * linear_mode must be SLA_LINEAR_MASK_PRODUCT (else SLA_ERR_UNSUPPORTED); branch dropping is
 * not available with it. */
int sla_forward_int8(const sla_problem* p, const void* Q, const void* K, const void* V,
                     const int32_t* idx, const float* alpha, float* O, void* ws, size_t ws_bytes,
                     hipStream_t stream);
int sla_forward_int8_ex(const sla_problem* p, const void* Q, const void* K, const void* V,
                        const int32_t* idx, const float* alpha, float* O, void* ws,
                        size_t ws_bytes, hipStream_t stream, const sla_forward_opts* opts);

/* Quantisation step of sla_forward_int8 on its own (byte-exact checks): int8 codes of X
 * [B][H][N][d] (bf16) to codes [B][H][N][d] and the per-block scales to scales [B][H][n_b]. */
int sla_quantize_int8(const sla_problem* p, const void* X, int8_t* codes, float* scales,
                      hipStream_t stream);

/* Quantisation step of sla_forward_fp8 on its own (for byte-exact checks): writes e4m3 codes
 * of X [B][H][N][d] (bf16) to codes [B][H][N][d] (uint8) and the per-block scales to
 * scales [B][H][n_b] (float32). */
int sla_quantize_e4m3(const sla_problem* p, const void* X, uint8_t* codes, float* scales,
                      hipStream_t stream);

/* Backward of the forward (the training path; SLA2 Italian summary section 2, Arabic summary
 * sections 2 and 2.jim: fine-tuning with the attention in place, the backward taken on the
 * unquantised values): gradients of O = alpha O_s + (1 - alpha) O_l with respect to Q, K, V and
 * alpha for the given kept sets (the HardTop-k router has no gradient).  dO [B][H][N][d] in the
 * dtype of Q; dQ, dK, dV [B][H][N][d] and dalpha [B][H][N] float32 outputs (overwritten).  The
 * forward is recomputed in the mask-product mode; O (optional, NULL to skip) receives it.  The
 * linear branch passes no gradient through rows where it is defined as 0 (empty unselected set
 * or zero denominator), and ReLU's derivative at 0 is taken as 0.  Only dtype SLA_BF16 with
 * d = 128 is compiled.  Needs sla_backward_workspace_bytes(p) bytes of workspace. */
size_t sla_backward_workspace_bytes(const sla_problem* p);
int sla_backward(const sla_problem* p, const void* Q, const void* K, const void* V,
                 const int32_t* idx, const float* alpha, const void* dO, float* dQ, float* dK,
                 float* dV, float* dalpha, float* O, void* ws, size_t ws_bytes,
                 hipStream_t stream);

/* Allocation-free router, for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): sla_route with the
 * workspace taken from a static device array of SLA_ROUTE_NOALLOC_SCRATCH_BYTES bytes inside
 * the library instead of an argument.  Each GPU the library runs on holds its own copy of the
 * array from the first call on it until the process ends; the call allocates nothing and calls
 * no allocating routine.  The array's address is looked up once per device, with that device
 * current, on its first call; call with the stream's device current (as torch does).  Every call
 * on a GPU shares that GPU's array (nothing in it needs to start at zero; the router overwrites
 * what it reads), so calls that overlap on one GPU (two streams, two threads) race: serialise
 * them.  A problem whose sla_route_workspace_bytes() exceeds the array gives
 * SLA_ERR_WORKSPACE (4 * B * H * n_b * d bf16 values plus alignment, e.g. B*H = 40 heads at
 * N = 75600, d = 128 need 48.4 MB).  Other arguments and errors as sla_route. */
#define SLA_ROUTE_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
int sla_route_noalloc(const sla_problem* p, const void* Q, const void* K, const float* proj_q,
                      const float* proj_k, int32_t* idx, uint8_t* mask, float* scores,
                      hipStream_t stream);

/* Debug check of an index list (HardTop-k's output: SLA2 Italian summary section 2.B, Arabic
 * summary section 2.ba): every entry of idx [B][H][n_b][topk] int32 lies in [0, n_b) and each
 * row is strictly ascending.  Runs one kernel on `stream`, then synchronises the stream (so
 * the host waits for everything enqueued before it) and returns SLA_OK, or SLA_ERR_INVALID for a
 * malformed list; topk = 0 checks nothing.  The result word is a file-scope device variable (one
 * per GPU): checks that overlap on one GPU race.
 * With SLA_VALIDATE=1 in the environment, sla_forward*, sla_backward and sla_pisa_forward run
 * this check first (after the host-side checks, after waiting for opts->idx_ready if given) and
 * return its SLA_ERR_INVALID with nothing else enqueued; this debug mode synchronises the host,
 * against the no-synchronisation rule above.  Without it, idx contents are trusted. */
int sla_validate_idx(const sla_problem* p, const int32_t* idx, hipStream_t stream);

const char* sla_status_string(int status);
/* hipError_t of the most recent SLA_ERR_HIP on the calling thread (0 if none). */
int sla_last_hip_error(void);

#ifdef __cplusplus
}
#endif

#endif /* SLA_H */
