// router.hip - the SLA2 router on gfx950 (SLA2 Italian summary section 2.B, Arabic summary
// sections 2.ba and 2.dal): block mean-pool of Q and K, learnable projections, block-score map
// and the inference-time HardTop-k.
//
//   pool_project_kernel  one workgroup per (8 blocks, head, Q|K): streams the block's rows
//                        (16-byte coalesced loads, fp32 sums), divides by the number of valid
//                        tokens, multiplies by W (fp32) and stores the result split into a
//                        bf16 high part and a bf16 low part (x = hi + lo + O(2^-17 |x|)).
//   score_topk_kernel    one workgroup per (16 query blocks, head): the 16 x n_b score tile
//                        s = (q~ . k~) / sqrt(d) by bf16 MFMA on the split operands
//                        (hi*hi + hi*lo + lo*hi, fp32 accumulation: about fp32 accuracy) into
//                        LDS (8 wavefronts, operand loads of two key tiles issued ahead of
//                        their MFMAs), then per row (one wavefront) the k-th largest score by
//                        a 32-step bitwise search on order-preserving keys (counts by ballot),
//                        and an ascending compaction that keeps the lowest indices among equal
//                        scores.
#include "sla_device.hpp"
#include "sla_launch.hpp"

namespace sla {

namespace {

constexpr int kPoolBlocksPerWg = 8;
constexpr int kPoolThreads = 256;

template <class T>
__device__ __forceinline__ void load_vec(const T* p, float* out);
template <>
__device__ __forceinline__ void load_vec<__bf16>(const __bf16* p, float* out) {
  bf16x8 v = *reinterpret_cast<const bf16x8*>(p);
#pragma unroll
  for (int i = 0; i < 8; ++i) out[i] = (float)v[i];
}
template <>
__device__ __forceinline__ void load_vec<float>(const float* p, float* out) {
  f32x4 v = *reinterpret_cast<const f32x4*>(p);
#pragma unroll
  for (int i = 0; i < 4; ++i) out[i] = v[i];
}

template <class T, int D>
__global__ __launch_bounds__(kPoolThreads) void pool_project_kernel(
    const T* __restrict__ Q, const T* __restrict__ K, const float* __restrict__ Wq,
    const float* __restrict__ Wk, int N, int nb, __bf16* __restrict__ q_hi,
    __bf16* __restrict__ q_lo, __bf16* __restrict__ k_hi, __bf16* __restrict__ k_lo) {
  constexpr int VEC = 16 / sizeof(T);      // elements per 16-byte load
  constexpr int TPR = D / VEC;             // threads per row
  constexpr int RPP = kPoolThreads / TPR;  // rows per pass
  static_assert(kBlock % RPP == 0, "rows per pass must divide the block");
  __shared__ float red[RPP][D];
  __shared__ float xbar[kPoolBlocksPerWg][D];

  const int tid = threadIdx.x;
  const int bh = blockIdx.y;
  const bool is_k = blockIdx.z != 0;
  const T* X = (is_k ? K : Q) + (size_t)bh * N * D;
  const float* W = is_k ? Wk : Wq;
  __bf16* out_hi = (is_k ? k_hi : q_hi) + (size_t)bh * nb * D;
  __bf16* out_lo = (is_k ? k_lo : q_lo) + (size_t)bh * nb * D;

  const int t0 = blockIdx.x * kPoolBlocksPerWg;
  const int nblk = min(kPoolBlocksPerWg, nb - t0);
  const int col = (tid % TPR) * VEC;
  const int roff = tid / TPR;

  // block b's rows: every load issued unconditionally (rows past N re-read the block's last
  // row and are dropped in the sum; a block past n_b re-reads the last block), and block b + 1's
  // loads go out before block b's sum, so each thread keeps two blocks' loads in flight
  float tmp[2][kBlock / RPP][VEC];
  auto load_block = [&](int b, float (&dst)[kBlock / RPP][VEC]) {
    const int row0 = min(t0 + b, nb - 1) * kBlock;
    const int last = min(kBlock, N - row0) - 1;
#pragma unroll
    for (int p = 0; p < kBlock / RPP; ++p)
      load_vec<T>(X + (size_t)(row0 + min(roff + p * RPP, last)) * D + col, dst[p]);
  };
  load_block(0, tmp[0]);
#pragma unroll
  for (int b = 0; b < kPoolBlocksPerWg; ++b) {
    if (b + 1 < kPoolBlocksPerWg) load_block(b + 1, tmp[(b + 1) & 1]);
    if (b < nblk) {
      const int cnt = min(kBlock, N - (t0 + b) * kBlock);
      float acc[VEC];
#pragma unroll
      for (int v = 0; v < VEC; ++v) acc[v] = 0.f;
#pragma unroll
      for (int p = 0; p < kBlock / RPP; ++p)
#pragma unroll
        for (int v = 0; v < VEC; ++v) acc[v] += roff + p * RPP < cnt ? tmp[b & 1][p][v] : 0.f;
#pragma unroll
      for (int v = 0; v < VEC; ++v) red[roff][col + v] = acc[v];
      __syncthreads();
      if (tid < D) {
        float sum = 0.f;
#pragma unroll
        for (int r = 0; r < RPP; ++r) sum += red[r][tid];
        xbar[b][tid] = sum / (float)cnt;
      }
      __syncthreads();
    }
  }

  // projection: y[b][c] = sum_r xbar[b][r] * W[r][c]; no W: the pooled means themselves
  constexpr int G = kPoolThreads / D;  // thread groups, each covering all D output columns
  const int c = tid % D;
  const int grp = tid / D;
  float y[kPoolBlocksPerWg / G];
  if (W) {
#pragma unroll
    for (int u = 0; u < kPoolBlocksPerWg / G; ++u) y[u] = 0.f;
#pragma unroll 32
    for (int r = 0; r < D; ++r) {
      const float w = W[r * D + c];
#pragma unroll
      for (int u = 0; u < kPoolBlocksPerWg / G; ++u) y[u] += xbar[grp + u * G][r] * w;
    }
  } else {
#pragma unroll
    for (int u = 0; u < kPoolBlocksPerWg / G; ++u) y[u] = xbar[grp + u * G][c];
  }
#pragma unroll
  for (int u = 0; u < kPoolBlocksPerWg / G; ++u) {
    const int b = grp + u * G;
    if (b < nblk) {
      const __bf16 hi = f2bf(y[u]);
      const __bf16 lo = f2bf(y[u] - bf2f(hi));
      out_hi[(size_t)(t0 + b) * D + c] = hi;
      out_lo[(size_t)(t0 + b) * D + c] = lo;
    }
  }
}

constexpr int kRowsPerWg = 16;   // query blocks per score/top-k workgroup (one MFMA row tile)
constexpr int kTopkThreads = 512;
constexpr int kTopkWaves = kTopkThreads / kWave;
constexpr int kMaxChunks = 32;   // n_b <= 2048

// Scores of 16 query blocks against all key blocks into LDS, then per row the k-th largest
// score and the ascending compaction.  NCH = key slots per lane (at least ceil(n_b / 64)):
// invalid slots hold key 0, below every valid key, so no slot needs a guard.  bias (optional,
// [bh][n_b]) is added to every score of key block j before the selection; probs receives the
// row softmax of the scores, or (raw) the scores themselves.
template <int D, int NCH>
__global__ __launch_bounds__(kTopkThreads) void score_topk_kernel(
    const __bf16* __restrict__ q_hi, const __bf16* __restrict__ q_lo,
    const __bf16* __restrict__ k_hi, const __bf16* __restrict__ k_lo, int nb, int topk,
    float scale, int nbp, const float* __restrict__ bias, int raw, int32_t* __restrict__ idx,
    uint8_t* __restrict__ mask, float* __restrict__ probs) {
  extern __shared__ float S[];  // [kRowsPerWg][nbp]
  const int lane = threadIdx.x % kWave;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);  // wavefront-uniform
  const int bh = blockIdx.y;
  const int i0 = blockIdx.x * kRowsPerWg;
  const size_t base = (size_t)bh * nb * D;

  // ---- scores: 16 x n_b tile, 16x16x32 MFMA on split operands (hi*hi + hi*lo + lo*hi) ----
  {
    constexpr int KS = D / 32;
    bf16x8 ahi[KS], alo[KS];
    const int arow = i0 + lane % 16;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const int col = 32 * s + 8 * (lane / 16);
      ahi[s] = arow < nb ? *reinterpret_cast<const bf16x8*>(q_hi + base + (size_t)arow * D + col) : bf16x8{};
      alo[s] = arow < nb ? *reinterpret_cast<const bf16x8*>(q_lo + base + (size_t)arow * D + col) : bf16x8{};
    }
    const int ntiles = (nb + 15) / 16;
    // two key tiles per step: all their operand loads are issued before the MFMAs
    for (int jt = wave; jt < ntiles; jt += 2 * kTopkWaves) {
      bf16x8 bhi[2][KS], blo[2][KS];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int j = (jt + u * kTopkWaves) * 16 + lane % 16;
#pragma unroll
        for (int s = 0; s < KS; ++s) {
          const int col = 32 * s + 8 * (lane / 16);
          bhi[u][s] = j < nb ? *reinterpret_cast<const bf16x8*>(k_hi + base + (size_t)j * D + col) : bf16x8{};
          blo[u][s] = j < nb ? *reinterpret_cast<const bf16x8*>(k_lo + base + (size_t)j * D + col) : bf16x8{};
        }
      }
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int t = jt + u * kTopkWaves;
        if (t >= ntiles) break;
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < KS; ++s) {
          acc = mfma16(alo[s], bhi[u][s], acc);
          acc = mfma16(ahi[s], blo[u][s], acc);
          acc = mfma16(ahi[s], bhi[u][s], acc);
        }
        const int j = t * 16 + lane % 16;
        const float bj = (bias && j < nb) ? bias[(size_t)bh * nb + j] : 0.f;
#pragma unroll
        for (int r = 0; r < 4; ++r) S[(4 * (lane / 16) + r) * nbp + j] = fmaf(acc[r], scale, bj);
      }
    }
  }
  __syncthreads();

  // ---- per row: k-th largest key, then ascending compaction ----
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int r = wave; r < kRowsPerWg; r += kTopkWaves) {
    const int i = i0 + r;
    if (i >= nb) break;
    const float* srow = S + r * nbp;
    u32 key[NCH];
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      const int j = c * kWave + lane;
      key[c] = j < nb ? float_key(srow[j]) : 0u;
    }
    // largest threshold T with count(key >= T) >= topk (all valid keys are >= 1)
    u32 T = 0xffffffffu;  // topk == 0: nothing is kept
    if (topk > 0) {
      T = 0;
      for (int bit = 31; bit >= 0; --bit) {
        const u32 cand = T | (1u << bit);
        int cnt = 0;
#pragma unroll
        for (int c = 0; c < NCH; ++c) cnt += __popcll(__ballot(key[c] >= cand));
        if (cnt >= topk) T = cand;
      }
    }
    int gt = 0;
#pragma unroll
    for (int c = 0; c < NCH; ++c) gt += __popcll(__ballot(key[c] > T));
    const int need = topk - gt;  // equal keys to keep, lowest index first
    int pos = 0, ties = 0;
    int32_t* irow = idx + ((size_t)bh * nb + i) * topk;
    uint8_t* mrow = mask ? mask + ((size_t)bh * nb + i) * nb : nullptr;
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      const int j = c * kWave + lane;
      const bool valid = j < nb;
      const bool eq = valid && topk > 0 && key[c] == T;
      const uint64_t eqm = __ballot(eq);
      const int rank = ties + __popcll(eqm & lt_mask);
      const bool sel = valid && topk > 0 && (key[c] > T || (eq && rank < need));
      const uint64_t selm = __ballot(sel);
      if (sel) irow[pos + __popcll(selm & lt_mask)] = j;
      if (mrow && valid) mrow[j] = sel ? 1 : 0;
      pos += __popcll(selm);
      ties += __popcll(eqm);
    }
    if (probs && raw) {
      float* prow = probs + ((size_t)bh * nb + i) * nb;
      for (int j = lane; j < nb; j += kWave) prow[j] = srow[j];
    } else if (probs) {
      float mx = -INFINITY;
      for (int j = lane; j < nb; j += kWave) mx = fmaxf(mx, srow[j]);
      mx = wave_max(mx);
      float sum = 0.f;
      for (int j = lane; j < nb; j += kWave) sum += __expf(srow[j] - mx);
      sum = wave_sum(sum);
      const float inv = 1.f / sum;
      float* prow = probs + ((size_t)bh * nb + i) * nb;
      for (int j = lane; j < nb; j += kWave) prow[j] = __expf(srow[j] - mx) * inv;
    }
  }
}

template <int D>
hipError_t launch_topk(const Dims& p, const __bf16* q_hi, const __bf16* q_lo,
                       const __bf16* k_hi, const __bf16* k_lo, const float* bias, int raw,
                       int32_t* idx, uint8_t* mask, float* probs, size_t lds,
                       hipStream_t stream) {
  const int nbp = (p.nb + 15) / 16 * 16;
  dim3 grid((p.nb + kRowsPerWg - 1) / kRowsPerWg, p.B * p.H);
  const float scale = 1.0f / sqrtf((float)D);
  const int nch = (p.nb + kWave - 1) / kWave;
  auto go = [&](auto kern) -> hipError_t {
    hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    kern<<<grid, kTopkThreads, lds, stream>>>(q_hi, q_lo, k_hi, k_lo, p.nb, p.topk, scale, nbp,
                                              bias, raw, idx, mask, probs);
    return hipGetLastError();
  };
  if (nch <= 1) return go(score_topk_kernel<D, 1>);
  if (nch <= 2) return go(score_topk_kernel<D, 2>);
  if (nch <= 4) return go(score_topk_kernel<D, 4>);
  if (nch <= 8) return go(score_topk_kernel<D, 8>);
  if (nch <= 16) return go(score_topk_kernel<D, 16>);
  if (nch <= 20) return go(score_topk_kernel<D, 20>);
  return go(score_topk_kernel<D, kMaxChunks>);
}

}  // namespace

size_t route_lds_bytes(int nb) {
  const int nbp = (nb + 15) / 16 * 16;
  return (size_t)kRowsPerWg * nbp * sizeof(float);
}

int route_max_blocks() { return kMaxChunks * kWave; }

hipError_t launch_route(const Dims& p, const void* Q, const void* K, const float* Wq,
                        const float* Wk, __bf16* q_hi, __bf16* q_lo, __bf16* k_hi,
                        __bf16* k_lo, int32_t* idx, uint8_t* mask, float* probs,
                        hipStream_t stream) {
  const int BH = p.B * p.H;
  dim3 g1((p.nb + kPoolBlocksPerWg - 1) / kPoolBlocksPerWg, BH, 2);
  if (p.dtype == kBF16 && p.d == 128)
    pool_project_kernel<__bf16, 128><<<g1, kPoolThreads, 0, stream>>>(
        (const __bf16*)Q, (const __bf16*)K, Wq, Wk, p.N, p.nb, q_hi, q_lo, k_hi, k_lo);
  else if (p.dtype == kBF16 && p.d == 64)
    pool_project_kernel<__bf16, 64><<<g1, kPoolThreads, 0, stream>>>(
        (const __bf16*)Q, (const __bf16*)K, Wq, Wk, p.N, p.nb, q_hi, q_lo, k_hi, k_lo);
  else if (p.dtype == kF32 && p.d == 128)
    pool_project_kernel<float, 128><<<g1, kPoolThreads, 0, stream>>>(
        (const float*)Q, (const float*)K, Wq, Wk, p.N, p.nb, q_hi, q_lo, k_hi, k_lo);
  else
    pool_project_kernel<float, 64><<<g1, kPoolThreads, 0, stream>>>(
        (const float*)Q, (const float*)K, Wq, Wk, p.N, p.nb, q_hi, q_lo, k_hi, k_lo);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;

  const size_t lds = route_lds_bytes(p.nb);
  if (p.d == 128)
    return launch_topk<128>(p, q_hi, q_lo, k_hi, k_lo, nullptr, 0, idx, mask, probs, lds, stream);
  return launch_topk<64>(p, q_hi, q_lo, k_hi, k_lo, nullptr, 0, idx, mask, probs, lds, stream);
}

hipError_t launch_pool_means(const Dims& p, const void* Q, const void* K, __bf16* q_hi,
                             __bf16* q_lo, __bf16* k_hi, __bf16* k_lo, hipStream_t stream) {
  // both tensors (grid z = 2), no projection
  dim3 g1((p.nb + kPoolBlocksPerWg - 1) / kPoolBlocksPerWg, p.B * p.H, 2);
  if (p.dtype == kBF16 && p.d == 128)
    pool_project_kernel<__bf16, 128><<<g1, kPoolThreads, 0, stream>>>(
        (const __bf16*)Q, (const __bf16*)K, nullptr, nullptr, p.N, p.nb, q_hi, q_lo, k_hi, k_lo);
  else if (p.dtype == kBF16 && p.d == 64)
    pool_project_kernel<__bf16, 64><<<g1, kPoolThreads, 0, stream>>>(
        (const __bf16*)Q, (const __bf16*)K, nullptr, nullptr, p.N, p.nb, q_hi, q_lo, k_hi, k_lo);
  else if (p.dtype == kF32 && p.d == 128)
    pool_project_kernel<float, 128><<<g1, kPoolThreads, 0, stream>>>(
        (const float*)Q, (const float*)K, nullptr, nullptr, p.N, p.nb, q_hi, q_lo, k_hi, k_lo);
  else
    pool_project_kernel<float, 64><<<g1, kPoolThreads, 0, stream>>>(
        (const float*)Q, (const float*)K, nullptr, nullptr, p.N, p.nb, q_hi, q_lo, k_hi, k_lo);
  return hipGetLastError();
}

hipError_t launch_pisa_route(const Dims& p, const void* Q, __bf16* q_hi, __bf16* q_lo,
                             const __bf16* kbar_hi, const __bf16* kbar_lo, const float* bias,
                             int32_t* idx, uint8_t* mask, float* scores, hipStream_t stream) {
  // pooled queries only (grid z = 1), no projection
  dim3 g1((p.nb + kPoolBlocksPerWg - 1) / kPoolBlocksPerWg, p.B * p.H, 1);
  if (p.dtype == kBF16 && p.d == 128)
    pool_project_kernel<__bf16, 128><<<g1, kPoolThreads, 0, stream>>>(
        (const __bf16*)Q, nullptr, nullptr, nullptr, p.N, p.nb, q_hi, q_lo, nullptr, nullptr);
  else if (p.dtype == kBF16 && p.d == 64)
    pool_project_kernel<__bf16, 64><<<g1, kPoolThreads, 0, stream>>>(
        (const __bf16*)Q, nullptr, nullptr, nullptr, p.N, p.nb, q_hi, q_lo, nullptr, nullptr);
  else if (p.dtype == kF32 && p.d == 128)
    pool_project_kernel<float, 128><<<g1, kPoolThreads, 0, stream>>>(
        (const float*)Q, nullptr, nullptr, nullptr, p.N, p.nb, q_hi, q_lo, nullptr, nullptr);
  else
    pool_project_kernel<float, 64><<<g1, kPoolThreads, 0, stream>>>(
        (const float*)Q, nullptr, nullptr, nullptr, p.N, p.nb, q_hi, q_lo, nullptr, nullptr);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const size_t lds = route_lds_bytes(p.nb);
  if (p.d == 128)
    return launch_topk<128>(p, q_hi, q_lo, kbar_hi, kbar_lo, bias, 1, idx, mask, scores, lds, stream);
  return launch_topk<64>(p, q_hi, q_lo, kbar_hi, kbar_lo, bias, 1, idx, mask, scores, lds, stream);
}

}  // namespace sla
