// soft.hip - the SoftTop-k training path of SLA2 on gfx950: the soft router, the gradients of
// the soft-mask forward with respect to the mask, and the stage-1 fit of proj_q, proj_k, alpha.
//
// SLA2 (Italian summary) section 2.B and (Arabic summary) section 2.ba: in training the router's
// mask comes from a differentiable SoftTop-k, so gradients reach proj_q and proj_k; (Arabic
// summary) section 2.dal: stage 1 fits the router and alpha by MSE against full attention.
// Reading (the pages leave SoftTop-k open): M_ij = sigmoid((s_ij - tau_i) / T) with tau_i such
// that sum_j M_ij = k; M weighs key block j in the sparse branch of query block i and 1 - M in
// its linear branch (0/1 gives the HardTop-k forward).
//
//   soft_pool_kernel     per (b, h, block, Q or K): the block mean in fp32 and its projection
//                        y = mean @ W (one thread per output channel).
//   soft_topk_kernel     per (b, h, query block): the score row s_ij = qt_i . kt_j / sqrt(d) in
//                        LDS, tau by bisection on sum_j sigmoid((s - tau) / T) = k (64 halvings
//                        of a bracket 60 T past the row's extremes), M and bf16(1 - M) (the
//                        weighted mask GEMM's operand, zero-padded).
//   soft_dm_sparse_kernel  per (b, h, query block) over every key block: S^T = K Q^T and
//                        dP^T = V dO_s^T on bf16 MFMA (wavefront w: keys 32 (w / 2) .. + 31,
//                        rows 32 (w % 2) .. + 31), then the tile sum of 2^(S c - lse2) (dP - D)
//                        per wavefront: the sparse branch's dM_ij in four parts.
//   soft_dm_linear_kernel  dM_ij of the linear branch, -(<dA_i, h_j> + dzeta_i . z_j): an MFMA
//                        product over the d*d state entries of the sliced bf16 dA_i^T and h_j^T
//                        (both row-contiguous in the entries, read straight from memory), plus
//                        the fp32 dzeta . z term.
//   soft_topk_bwd_kernel per row: dM = the parts summed, ds = (M(1-M)/T)(dM - sum dM M(1-M) /
//                        sum M(1-M)).
//   router_rows_kernel   dqt_i = sum_j ds_ij kt_j / sqrt(d), dkt_j = sum_i ds_ij qt_i / sqrt(d).
//   proj_grad_kernel     dW[r][c] = sum over every (b, h, block) of xbar[r] dy[c]: partial sums
//                        over 64 chunks of the rows, added in order by proj_grad_sum_kernel.
//   soft_loss_kernel / soft_loss_sum_kernel / soft_update_kernel  the stage-1 loss, dO and the
//                        step W -= lr dW, alpha = clamp(alpha - lr dalpha, 0, 1).
// bf16 Q, K, V with d = 128; everything else fp32.  No float atomics: every sum has a fixed
// order, so a step is deterministic.
#include "sla_device.hpp"
#include "sla_launch.hpp"
#include "sla_tiles.hpp"

namespace sla {

namespace {

constexpr int kSoftD = 128;
constexpr int kLossThreads = 256;
constexpr int kLossPerThread = 16;

__device__ __forceinline__ float block_sum256(float v, float* red) {
  v = wave_sum(v);
  const int w = threadIdx.x / kWave;
  __syncthreads();
  if (threadIdx.x % kWave == 0) red[w] = v;
  __syncthreads();
  return red[0] + red[1] + red[2] + red[3];
}
__device__ __forceinline__ float block_max256(float v, float* red) {
  v = wave_max(v);
  const int w = threadIdx.x / kWave;
  __syncthreads();
  if (threadIdx.x % kWave == 0) red[w] = v;
  __syncthreads();
  return fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
}
__device__ __forceinline__ float sigmoidf_(float u) { return 1.f / (1.f + __expf(-u)); }

__global__ __launch_bounds__(kSoftD) void soft_pool_kernel(const __bf16* __restrict__ Q,
                                                           const __bf16* __restrict__ K,
                                                           const float* __restrict__ Wq,
                                                           const float* __restrict__ Wk, int N,
                                                           int nb, float* __restrict__ qbar,
                                                           float* __restrict__ kbar,
                                                           float* __restrict__ qt,
                                                           float* __restrict__ kt) {
  constexpr int D = kSoftD;
  __shared__ float xs[D];
  const int c = threadIdx.x, t = blockIdx.x, bh = blockIdx.y, which = blockIdx.z;
  const __bf16* X = (which ? K : Q) + ((size_t)bh * N + (size_t)t * kBlock) * D;
  const float* W = which ? Wk : Wq;
  const int cnt = min(kBlock, N - t * kBlock);
  float sum = 0.f;
  for (int r = 0; r < cnt; ++r) sum += bf2f(X[(size_t)r * D + c]);
  const float mean = sum / (float)cnt;
  xs[c] = mean;
  __syncthreads();
  float y = 0.f;
  for (int r = 0; r < D; ++r) y = fmaf(xs[r], W[r * D + c], y);
  const size_t o = ((size_t)bh * nb + t) * D + c;
  (which ? kbar : qbar)[o] = mean;
  (which ? kt : qt)[o] = y;
}

__global__ __launch_bounds__(256) void soft_topk_kernel(const float* __restrict__ qt,
                                                        const float* __restrict__ kt, int nb,
                                                        int topk, float inv_sqrt_d, float temp,
                                                        int pitch, float* __restrict__ M,
                                                        __bf16* __restrict__ wt) {
  constexpr int D = kSoftD;
  __shared__ float qs[D];
  __shared__ float srow[2048];
  __shared__ float red[4];
  const int tid = threadIdx.x, i = blockIdx.x, bh = blockIdx.y;
  if (tid < D) qs[tid] = qt[((size_t)bh * nb + i) * D + tid];
  __syncthreads();
  float mn = INFINITY, mx = -INFINITY;
  for (int j = tid; j < nb; j += 256) {
    const f32x4* kr = reinterpret_cast<const f32x4*>(kt + ((size_t)bh * nb + j) * D);
    float s = 0.f;
#pragma unroll 8
    for (int c4 = 0; c4 < D / 4; ++c4) {
      const f32x4 k4 = kr[c4];
#pragma unroll
      for (int e = 0; e < 4; ++e) s = fmaf(qs[4 * c4 + e], k4[e], s);
    }
    s *= inv_sqrt_d;
    srow[j] = s;
    mn = fminf(mn, s);
    mx = fmaxf(mx, s);
  }
  mn = -block_max256(-mn, red);
  mx = block_max256(mx, red);
  float tau = 0.f;
  const bool all = topk >= nb, none = topk <= 0;
  if (!all && !none) {
    float lo = mn - 60.f * temp, hi = mx + 60.f * temp;
    const float inv_t = 1.f / temp;
    for (int it = 0; it < 64; ++it) {
      const float mid = 0.5f * (lo + hi);
      float tot = 0.f;
      for (int j = tid; j < nb; j += 256) tot += sigmoidf_((srow[j] - mid) * inv_t);
      tot = block_sum256(tot, red);
      if (tot > (float)topk) lo = mid;  // the threshold is too low: raise it
      else hi = mid;
    }
    tau = 0.5f * (lo + hi);
  }
  const float inv_t = 1.f / temp;
  float* mrow = M + ((size_t)bh * nb + i) * nb;
  __bf16* wrow = wt + ((size_t)bh * nb + i) * pitch;
  for (int j = tid; j < pitch; j += 256) {
    if (j < nb) {
      const float m = all ? 1.f : (none ? 0.f : sigmoidf_((srow[j] - tau) * inv_t));
      mrow[j] = m;
      wrow[j] = f2bf(1.f - m);
    } else {
      wrow[j] = f2bf(0.f);
    }
  }
}

// dM of the sparse branch.  One workgroup per (b, h, query block); the key tiles are staged like
// the forward's (direct buffer loads into the swizzled row layout, double-buffered).
__global__ __launch_bounds__(256, 2) void soft_dm_sparse_kernel(
    const __bf16* __restrict__ Q, const __bf16* __restrict__ K, const __bf16* __restrict__ V,
    const __bf16* __restrict__ dOs, const float* __restrict__ lse2, const float* __restrict__ Dr,
    int N, int nb, float c_log2, float* __restrict__ dmsp) {
  constexpr int D = kSoftD, NS = D / 16, TILE = kBlock * D;
  __shared__ __attribute__((aligned(16))) __bf16 kb0[TILE];
  __shared__ __attribute__((aligned(16))) __bf16 kb1[TILE];
  __shared__ __attribute__((aligned(16))) __bf16 vb0[TILE];
  __shared__ __attribute__((aligned(16))) __bf16 vb1[TILE];
  const int tid = threadIdx.x, lane = tid % kWave, g = lane / 32;
  const int w = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int i = blockIdx.x, bh = blockIdx.y;
  const size_t hoff = (size_t)bh * N * D;
  const __amdgpu_buffer_rsrc_t rk = make_rsrc(K + hoff, (uint32_t)((size_t)N * D * 2));
  const __amdgpu_buffer_rsrc_t rv = make_rsrc(V + hoff, (uint32_t)((size_t)N * D * 2));
  const uint32_t lane_voff = tile_lane_voff<256>(tid);
  auto stage = [&](int j, int buf) {
    const uint32_t toff = (uint32_t)j * (uint32_t)(TILE * 2);
    load_tile_buf<256>(rk, lane_voff, toff, buf ? kb1 : kb0, tid, (j + 1) * kBlock > N);
    load_tile_buf<256>(rv, lane_voff, toff, buf ? vb1 : vb0, tid, (j + 1) * kBlock > N);
  };
  // this wavefront's 32 query rows (B operands) and keys 32 (w / 2) .. + 31 of every tile
  const int row = i * kBlock + 32 * (w % 2) + lane % 32;
  const bool row_ok = row < N;
  const int rr = min(row, N - 1);
  bf16x8 q[NS], go[NS];
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    q[s] = row_ok ? *reinterpret_cast<const bf16x8*>(Q + hoff + (size_t)rr * D + 16 * s + 8 * g) : bf16x8{};
    go[s] = row_ok ? *reinterpret_cast<const bf16x8*>(dOs + hoff + (size_t)rr * D + 16 * s + 8 * g) : bf16x8{};
  }
  const float l2 = row_ok ? lse2[(size_t)bh * N + rr] : INFINITY;
  const float dr = row_ok ? Dr[(size_t)bh * N + rr] : 0.f;
  const int kh = 32 * (w / 2);
  const int ap_row = row_part(lane);
  stage(0, 0);
  wait_vmem();
  __syncthreads();
  for (int j = 0; j < nb; ++j) {
    const int buf = j & 1;
    if (j + 1 < nb) stage(j + 1, buf ^ 1);
    const __bf16* Ks = buf ? kb1 : kb0;
    const __bf16* Vs = buf ? vb1 : vb0;
    f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
    for (int k = 0; k < NS; ++k) {
      const int off = kh * 256 + (ap_row ^ (32 * k));
      s = mfma32(lds_row16(Ks, off), q[k], s);
      dp = mfma32(lds_row16(Vs, off), go[k], dp);
    }
    const int nv = min(kBlock, N - j * kBlock);
    float acc = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int key = kh + 8 * (r / 4) + 4 * g + r % 4;
      const float p = key < nv ? fast_exp2(fmaf(s[r], c_log2, -l2)) : 0.f;
      acc = fmaf(p, dp[r] - dr, acc);
    }
    acc = wave_sum(acc);
    if (lane == 0) dmsp[(((size_t)bh * nb + i) * nb + j) * 4 + w] = acc;
    wait_vmem();
    __syncthreads();
  }
}

// dM of the linear branch: C[i][j] = <dA_i, h_j> over the d*d entries (sliced bf16 layout
// [BH][d*d/64][nb][64], entry e = 64 sl + t), minus-signed with the dzeta . z term.  Workgroup:
// 64 query blocks x 64 key blocks; wavefront w: query half w % 2, key half w / 2.
__global__ __launch_bounds__(256) void soft_dm_linear_kernel(const __bf16* __restrict__ dA,
                                                             const __bf16* __restrict__ hj,
                                                             const float* __restrict__ dzeta,
                                                             const float* __restrict__ zb, int nb,
                                                             float* __restrict__ dmlin) {
  constexpr int D = kSoftD, SL = D * D / 64;
  const int tid = threadIdx.x, lane = tid % kWave, g = lane / 32, w = tid / kWave;
  const int bh = blockIdx.z;
  const int i0 = blockIdx.x * 64 + 32 * (w % 2), j0 = blockIdx.y * 64 + 32 * (w / 2);
  const int ia = min(i0 + lane % 32, nb - 1), jb = min(j0 + lane % 32, nb - 1);
  const __bf16* abase = dA + ((size_t)bh * SL * nb + ia) * 64 + 8 * g;
  const __bf16* bbase = hj + ((size_t)bh * SL * nb + jb) * 64 + 8 * g;
  f32x16 acc = f32x16{};
  for (int sl = 0; sl < SL; ++sl) {
    const size_t so = (size_t)sl * nb * 64;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(abase + so + 16 * ks);
      const bf16x8 b = *reinterpret_cast<const bf16x8*>(bbase + so + 16 * ks);
      acc = mfma32(a, b, acc);
    }
  }
  // lane holds C[i0 + 8 (r / 4) + 4 g + r % 4][j0 + lane % 32]
  const int j = j0 + lane % 32;
  if (j >= nb) return;
  const float* zr = zb + ((size_t)bh * nb + j) * D;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int ii = i0 + 8 * (r / 4) + 4 * g + r % 4;
    if (ii >= nb) continue;
    const float* dz = dzeta + ((size_t)bh * nb + ii) * D;
    float zt = 0.f;
    for (int c = 0; c < D; ++c) zt = fmaf(dz[c], zr[c], zt);
    dmlin[((size_t)bh * nb + ii) * nb + j] = -(acc[r] + zt);
  }
}

// wt = bf16(1 - M), zero past n_b (the weighted mask GEMM's operand)
__global__ __launch_bounds__(256) void soft_weights_kernel(const float* __restrict__ M, int nb,
                                                           int pitch, __bf16* __restrict__ wt) {
  const int i = blockIdx.x, bh = blockIdx.y;
  const float* mrow = M + ((size_t)bh * nb + i) * nb;
  __bf16* wrow = wt + ((size_t)bh * nb + i) * pitch;
  for (int j = threadIdx.x; j < pitch; j += 256) wrow[j] = f2bf(j < nb ? 1.f - mrow[j] : 0.f);
}

__global__ __launch_bounds__(256) void soft_topk_bwd_kernel(const float* __restrict__ M,
                                                            const float* __restrict__ dmsp,
                                                            const float* __restrict__ dmlin,
                                                            int nb, int topk, float temp,
                                                            float* __restrict__ ds,
                                                            float* __restrict__ dM_out) {
  __shared__ float red[4];
  const int tid = threadIdx.x, i = blockIdx.x, bh = blockIdx.y;
  const size_t row = ((size_t)bh * nb + i) * nb;
  float ssp = 0.f, sdm = 0.f;
  for (int j = tid; j < nb; j += 256) {
    const f32x4 p = *reinterpret_cast<const f32x4*>(dmsp + (row + j) * 4);
    const float dm = (p[0] + p[1]) + (p[2] + p[3]) + dmlin[row + j];
    const float m = M[row + j], sp = m * (1.f - m);
    ssp += sp;
    sdm = fmaf(dm, sp, sdm);
  }
  ssp = block_sum256(ssp, red);
  sdm = block_sum256(sdm, red);
  const bool live = topk > 0 && topk < nb && ssp > 0.f;
  const float corr = live ? sdm / ssp : 0.f, inv_t = 1.f / temp;
  for (int j = tid; j < nb; j += 256) {
    const f32x4 p = *reinterpret_cast<const f32x4*>(dmsp + (row + j) * 4);
    const float dm = (p[0] + p[1]) + (p[2] + p[3]) + dmlin[row + j];
    const float m = M[row + j];
    ds[row + j] = live ? m * (1.f - m) * inv_t * (dm - corr) : 0.f;
    if (dM_out) dM_out[row + j] = dm;
  }
}

__global__ __launch_bounds__(kSoftD) void router_rows_kernel(const float* __restrict__ ds,
                                                             const float* __restrict__ qt,
                                                             const float* __restrict__ kt, int nb,
                                                             float inv_sqrt_d,
                                                             float* __restrict__ dqt,
                                                             float* __restrict__ dkt) {
  constexpr int D = kSoftD;
  constexpr int U = 8;  // independent partial sums (loads in flight), added in a fixed order
  const int c = threadIdx.x, r = blockIdx.x, bh = blockIdx.y, which = blockIdx.z;
  const float* dsh = ds + (size_t)bh * nb * nb;
  // which 0: dqt_r = sum_j ds[r][j] kt_j; which 1: dkt_r = sum_i ds[i][r] qt_i
  const float* other = (which == 0 ? kt : qt) + (size_t)bh * nb * D;
  const size_t sstride = which == 0 ? 1 : (size_t)nb;
  const float* srow = dsh + (which == 0 ? (size_t)r * nb : (size_t)r);
  float acc[U];
#pragma unroll
  for (int u = 0; u < U; ++u) acc[u] = 0.f;
  int j = 0;
  for (; j + U <= nb; j += U)
#pragma unroll
    for (int u = 0; u < U; ++u) acc[u] = fmaf(srow[(size_t)(j + u) * sstride], other[(size_t)(j + u) * D + c], acc[u]);
  for (; j < nb; ++j) acc[0] = fmaf(srow[(size_t)j * sstride], other[(size_t)j * D + c], acc[0]);
  float sum = 0.f;
#pragma unroll
  for (int u = 0; u < U; ++u) sum += acc[u];
  (which == 0 ? dqt : dkt)[((size_t)bh * nb + r) * D + c] = sum * inv_sqrt_d;
}

// dW = x^T dy over `rows` rows in chunks: part[which][chunk][r][c] = sum over the chunk's rows
// of x[t][r] dy[t][c] (four partial sums in flight), then proj_grad_sum_kernel adds the chunks in
// order
constexpr int kProjChunks = 64;

__global__ __launch_bounds__(kSoftD) void proj_grad_kernel(const float* __restrict__ qbar,
                                                           const float* __restrict__ kbar,
                                                           const float* __restrict__ dqt,
                                                           const float* __restrict__ dkt, int rows,
                                                           int per_chunk, float* __restrict__ part) {
  constexpr int D = kSoftD;
  const int c = threadIdx.x, r = blockIdx.x, which = blockIdx.y, ch = blockIdx.z;
  const float* x = which ? kbar : qbar;
  const float* dy = which ? dkt : dqt;
  const int t0 = ch * per_chunk, t1 = min(rows, t0 + per_chunk);
  float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;
  int t = t0;
  for (; t + 4 <= t1; t += 4) {
    a0 = fmaf(x[(size_t)t * D + r], dy[(size_t)t * D + c], a0);
    a1 = fmaf(x[(size_t)(t + 1) * D + r], dy[(size_t)(t + 1) * D + c], a1);
    a2 = fmaf(x[(size_t)(t + 2) * D + r], dy[(size_t)(t + 2) * D + c], a2);
    a3 = fmaf(x[(size_t)(t + 3) * D + r], dy[(size_t)(t + 3) * D + c], a3);
  }
  for (; t < t1; ++t) a0 = fmaf(x[(size_t)t * D + r], dy[(size_t)t * D + c], a0);
  part[(((size_t)which * kProjChunks + ch) * D + r) * D + c] = (a0 + a1) + (a2 + a3);
}

__global__ __launch_bounds__(kSoftD) void proj_grad_sum_kernel(const float* __restrict__ part,
                                                               float* __restrict__ dWq,
                                                               float* __restrict__ dWk) {
  constexpr int D = kSoftD;
  const int c = threadIdx.x, r = blockIdx.x, which = blockIdx.y;
  float acc = 0.f;
  for (int ch = 0; ch < kProjChunks; ++ch) acc += part[(((size_t)which * kProjChunks + ch) * D + r) * D + c];
  (which ? dWk : dWq)[r * D + c] = acc;
}

__global__ __launch_bounds__(kLossThreads) void soft_loss_kernel(const float* __restrict__ O,
                                                                 const float* __restrict__ Of,
                                                                 size_t count, float scale,
                                                                 __bf16* __restrict__ dO,
                                                                 float* __restrict__ parts) {
  __shared__ float red[4];
  const size_t base = (size_t)blockIdx.x * kLossThreads * kLossPerThread;
  float acc = 0.f;
#pragma unroll
  for (int u = 0; u < kLossPerThread; ++u) {
    const size_t e = base + (size_t)u * kLossThreads + threadIdx.x;
    if (e < count) {
      const float dlt = O[e] - Of[e];
      dO[e] = f2bf(scale * dlt);
      acc = fmaf(dlt, dlt, acc);
    }
  }
  acc = block_sum256(acc, red);
  if (threadIdx.x == 0) parts[blockIdx.x] = acc;
}

__global__ __launch_bounds__(256) void soft_loss_sum_kernel(const float* __restrict__ parts, int n,
                                                            float inv_count, float* __restrict__ loss) {
  __shared__ float red[4];
  float acc = 0.f;
  for (int t = threadIdx.x; t < n; t += 256) acc += parts[t];
  acc = block_sum256(acc, red);
  if (threadIdx.x == 0) loss[0] = acc * inv_count;
}

__global__ __launch_bounds__(256) void soft_update_kernel(float* __restrict__ Wq, float* __restrict__ Wk,
                                                          float* __restrict__ alpha,
                                                          const float* __restrict__ dWq,
                                                          const float* __restrict__ dWk,
                                                          const float* __restrict__ dalpha, int nw,
                                                          size_t na, float lr_w, float lr_a) {
  const size_t t = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (t < (size_t)nw) {
    Wq[t] -= lr_w * dWq[t];
    Wk[t] -= lr_w * dWk[t];
  }
  if (t < na) alpha[t] = fminf(fmaxf(alpha[t] - lr_a * dalpha[t], 0.f), 1.f);
}

}  // namespace

hipError_t launch_soft_pool(const Dims& p, const void* Q, const void* K, const float* Wq,
                            const float* Wk, float* qbar, float* kbar, float* qt, float* kt,
                            hipStream_t stream) {
  if (p.d != kSoftD || p.dtype != kBF16) return hipErrorInvalidValue;
  soft_pool_kernel<<<dim3(p.nb, p.B * p.H, 2), kSoftD, 0, stream>>>(
      (const __bf16*)Q, (const __bf16*)K, Wq, Wk, p.N, p.nb, qbar, kbar, qt, kt);
  return hipGetLastError();
}

hipError_t launch_soft_topk(const Dims& p, const float* qt, const float* kt, float temp, float* M,
                            __bf16* wt, hipStream_t stream) {
  if (p.d != kSoftD || p.nb > 2048) return hipErrorInvalidValue;
  soft_topk_kernel<<<dim3(p.nb, p.B * p.H), 256, 0, stream>>>(
      qt, kt, p.nb, p.topk, 1.f / sqrtf((float)kSoftD), temp, tsel_weight_pitch(p.nb), M, wt);
  return hipGetLastError();
}

hipError_t launch_soft_weights(const Dims& p, const float* M, __bf16* wt, hipStream_t stream) {
  soft_weights_kernel<<<dim3(p.nb, p.B * p.H), 256, 0, stream>>>(M, p.nb, tsel_weight_pitch(p.nb), wt);
  return hipGetLastError();
}

hipError_t launch_soft_dm_sparse(const Dims& p, const void* Q, const void* K, const void* V,
                                 const __bf16* dOs, const float* lse2, const float* Dr, float* dmsp,
                                 hipStream_t stream) {
  if (p.d != kSoftD || p.dtype != kBF16) return hipErrorInvalidValue;
  soft_dm_sparse_kernel<<<dim3(p.nb, p.B * p.H), 256, 0, stream>>>(
      (const __bf16*)Q, (const __bf16*)K, (const __bf16*)V, dOs, lse2, Dr, p.N, p.nb,
      1.4426950408889634f / sqrtf((float)kSoftD), dmsp);
  return hipGetLastError();
}

hipError_t launch_soft_dm_linear(const Dims& p, const __bf16* dA_bf, const __bf16* hj_bf,
                                 const float* dzeta, const float* zb, float* dmlin,
                                 hipStream_t stream) {
  if (p.d != kSoftD) return hipErrorInvalidValue;
  const int t = (p.nb + 63) / 64;
  soft_dm_linear_kernel<<<dim3(t, t, p.B * p.H), 256, 0, stream>>>(dA_bf, hj_bf, dzeta, zb, p.nb, dmlin);
  return hipGetLastError();
}

hipError_t launch_soft_topk_bwd(const Dims& p, const float* M, const float* dmsp, const float* dmlin,
                                float temp, float* ds, float* dM_out, hipStream_t stream) {
  soft_topk_bwd_kernel<<<dim3(p.nb, p.B * p.H), 256, 0, stream>>>(M, dmsp, dmlin, p.nb, p.topk, temp,
                                                                   ds, dM_out);
  return hipGetLastError();
}

size_t router_bwd_part_floats() { return (size_t)2 * kProjChunks * kSoftD * kSoftD; }

hipError_t launch_router_bwd(const Dims& p, const float* ds, const float* qbar, const float* kbar,
                             const float* qt, const float* kt, float* dqt, float* dkt, float* dWq,
                             float* dWk, float* part, hipStream_t stream) {
  if (p.d != kSoftD) return hipErrorInvalidValue;
  router_rows_kernel<<<dim3(p.nb, p.B * p.H, 2), kSoftD, 0, stream>>>(ds, qt, kt, p.nb,
                                                                       1.f / sqrtf((float)kSoftD), dqt, dkt);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int rows = p.B * p.H * p.nb;
  const int per_chunk = (rows + kProjChunks - 1) / kProjChunks;
  proj_grad_kernel<<<dim3(kSoftD, 2, kProjChunks), kSoftD, 0, stream>>>(qbar, kbar, dqt, dkt, rows, per_chunk,
                                                                       part);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  proj_grad_sum_kernel<<<dim3(kSoftD, 2), kSoftD, 0, stream>>>(part, dWq, dWk);
  return hipGetLastError();
}

int soft_loss_parts(const Dims& p) {
  const size_t count = (size_t)p.B * p.H * p.N * p.d;
  const size_t per = (size_t)kLossThreads * kLossPerThread;
  return (int)((count + per - 1) / per);
}

hipError_t launch_soft_loss(const Dims& p, const float* O, const float* O_full, __bf16* dO,
                            float* parts, float* loss, hipStream_t stream) {
  const size_t count = (size_t)p.B * p.H * p.N * p.d;
  const int np = soft_loss_parts(p);
  soft_loss_kernel<<<np, kLossThreads, 0, stream>>>(O, O_full, count, 2.f / (float)count, dO, parts);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  soft_loss_sum_kernel<<<1, 256, 0, stream>>>(parts, np, 1.f / (float)count, loss);
  return hipGetLastError();
}

hipError_t launch_soft_update(const Dims& p, float* Wq, float* Wk, float* alpha, const float* dWq,
                              const float* dWk, const float* dalpha, float lr_w, float lr_a,
                              hipStream_t stream) {
  const int nw = p.d * p.d;
  const size_t na = (size_t)p.B * p.H * p.N;
  const size_t n = na > (size_t)nw ? na : (size_t)nw;
  soft_update_kernel<<<(unsigned)((n + 255) / 256), 256, 0, stream>>>(Wq, Wk, alpha, dWq, dWk, dalpha, nw,
                                                                       na, lr_w, lr_a);
  return hipGetLastError();
}

}  // namespace sla
