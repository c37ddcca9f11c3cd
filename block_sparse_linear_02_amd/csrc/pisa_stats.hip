// pisa_stats.hip - the per-key-block statistics of PISA on gfx950.
//
// Source: "PISA - Piecewise Sparse Attention per Efficient Diffusion Transformers", Italian
// technical summary, section 2: the pre-computation phase of the fused kernel (block centroids,
// value sums, the global statistic Hbar = mean over all blocks of the per-block first-order
// matrices) and the covariance-aware routing score M_j = ||H_j - Hbar||.  For key block j with
// valid tokens n (r_j of them), centroid kbar_j = mean_n k_n and value sum vs_j = sum_n v_n:
//   H_j = sum_n (k_n - kbar_j)^T v_n = K_j^T V_j - kbar_j^T vs_j   [d x d, K channel x V channel]
// (the first-order Taylor term of the block around its centroid), M_j its Frobenius distance
// from Hbar.
//
//   pisa_stats_kernel<PASS 0>  one workgroup per (chunk of key blocks, head), 256 threads.  Each
//                        64-token tile of K and V is streamed with 16-byte coalesced loads (the
//                        next tile's loads in flight while the current one is used); the column
//                        sums come from the loaded registers in fp32 (exact inputs, fp32 inputs
//                        unrounded), the tiles go to LDS as bf16 and V^T K is accumulated on
//                        bf16 MFMA (fp32 accumulation; bf16 inputs make every product exact),
//                        then the rank-one term vs_j kbar_j is subtracted in fp32 from the
//                        accumulators.  Writes kbar_j (bf16 hi + lo, x = hi + lo + O(2^-17 |x|))
//                        and vs_j (bf16) per block, and the chunk's sum of H_j^T / n_b.
//   reduce_kernel        (linear_state.hip) sums the chunk partials in a fixed order: Hbar^T in
//                        bf16 [c][c'] for the forward's MFMA and Hbar in fp32 [c'][c].
//   pisa_stats_kernel<PASS 1>  recomputes every H_j the same way (re-reading K and V costs 32 KB
//                        per block, less than storing and re-reading H_j), subtracts Hbar
//                        (held in registers for the whole chunk), and writes M_j and ln M_j
//                        (ln 0 = -inf: a block that equals the mean is never preferred).
#include "sla_device.hpp"
#include "sla_launch.hpp"
#include "sla_tiles.hpp"

namespace sla {

namespace {

constexpr int kStatThreads = 256;

template <class T>
__device__ __forceinline__ void unpack16(i32x4 r, float* out);
template <>
__device__ __forceinline__ void unpack16<__bf16>(i32x4 r, float* out) {
  const bf16x8 v = __builtin_bit_cast(bf16x8, r);
#pragma unroll
  for (int e = 0; e < 8; ++e) out[e] = bf2f(v[e]);
}
template <>
__device__ __forceinline__ void unpack16<float>(i32x4 r, float* out) {
  const f32x4 v = __builtin_bit_cast(f32x4, r);
#pragma unroll
  for (int e = 0; e < 4; ++e) out[e] = v[e];
}

template <class T, int D, int PASS>
__global__ __launch_bounds__(kStatThreads) void pisa_stats_kernel(
    const T* __restrict__ K, const T* __restrict__ V, int N, int nb, int cb,
    __bf16* __restrict__ kbar_hi, __bf16* __restrict__ kbar_lo, __bf16* __restrict__ vsum,
    float* __restrict__ h_part, const float* __restrict__ hbar, float* __restrict__ Mout,
    float* __restrict__ lnM) {
  using LD = TileLoader<T, D, kStatThreads>;
  constexpr int VEC = LD::VEC, CPR = LD::CPR;
  constexpr int RG = kStatThreads / CPR;  // row groups: thread t loads rows t / CPR + RG u
  static_assert(kStatThreads % CPR == 0, "a thread's chunks must share one column chunk");
  static_assert(2 * D <= kStatThreads, "one thread per centroid and per value-sum channel");
  constexpr int NT = D / 64;  // 32x32 output tiles per wave per dimension
  __shared__ __attribute__((aligned(16))) __bf16 Ks[TileLayout<D>::ELEMS];
  __shared__ __attribute__((aligned(16))) __bf16 Vs[TileLayout<D>::ELEMS];
  __shared__ float red[2][RG][D];  // column partial sums of the K and V tiles
  __shared__ float kb[D], vb[D];   // kbar_j and vs_j of the current block (fp32)
  __shared__ float sqw[kStatThreads / kWave];

  const int tid = threadIdx.x;
  const int lane = tid % kWave, g = lane / 32;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int bh = blockIdx.y, chunk = blockIdx.x;
  const int j0 = chunk * cb;
  const int j1 = min(nb, j0 + cb);
  const T* Kb = K + (size_t)bh * N * D;
  const T* Vb = V + (size_t)bh * N * D;
  // wave -> rows c (V channels) r0 .., columns c' (K channels) c0 .. of H^T
  const int r0 = (wave / 2) * 32 * NT;
  const int c0 = (wave % 2) * 32 * NT;
  const float inv_nb = 1.f / (float)nb;

  f32x16 acc[NT][NT];
#pragma unroll
  for (int a = 0; a < NT; ++a)
#pragma unroll
    for (int b = 0; b < NT; ++b) acc[a][b] = f32x16{};
  // PASS 1: Hbar^T at this lane's accumulator positions (Hbar is stored [c'][c])
  f32x16 hb[PASS == 1 ? NT : 1][PASS == 1 ? NT : 1];
  if constexpr (PASS == 1) {
    const float* hp = hbar + (size_t)bh * D * D;
#pragma unroll
    for (int a = 0; a < NT; ++a)
#pragma unroll
      for (int b = 0; b < NT; ++b)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int c = r0 + 32 * a + 8 * (i / 4) + 4 * g + i % 4;
          const int cp = c0 + 32 * b + lane % 32;
          hb[a][b][i] = hp[(size_t)cp * D + c];
        }
  }

  LD lk, lv;
  lk.load(Kb + (size_t)j0 * kBlock * D, min(kBlock, N - j0 * kBlock), tid);
  lv.load(Vb + (size_t)j0 * kBlock * D, min(kBlock, N - j0 * kBlock), tid);

  for (int j = j0; j < j1; ++j) {
    const int cnt = min(kBlock, N - j * kBlock);
    __syncthreads();  // the previous block's tiles, sums and statistics are consumed
    lk.store(Ks, tid);
    lv.store(Vs, tid);
    {
      // column sums of the loaded rows (rows past the block read as zero)
      float sk[VEC], sv[VEC];
#pragma unroll
      for (int e = 0; e < VEC; ++e) sk[e] = sv[e] = 0.f;
#pragma unroll
      for (int u = 0; u < LD::PER; ++u) {
        float xk[VEC], xv[VEC];
        unpack16<T>(lk.r[u], xk);
        unpack16<T>(lv.r[u], xv);
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
          sk[e] += xk[e];
          sv[e] += xv[e];
        }
      }
      const int col = (tid % CPR) * VEC, rg = tid / CPR;
#pragma unroll
      for (int e = 0; e < VEC; ++e) {
        red[0][rg][col + e] = sk[e];
        red[1][rg][col + e] = sv[e];
      }
    }
    __syncthreads();
    if (j + 1 < j1) {
      const int nv = min(kBlock, N - (j + 1) * kBlock);
      lk.load(Kb + (size_t)(j + 1) * kBlock * D, nv, tid);
      lv.load(Vb + (size_t)(j + 1) * kBlock * D, nv, tid);
    }
    if (tid < 2 * D) {
      const int part = tid / D, c = tid % D;
      float s = 0.f;
#pragma unroll
      for (int r = 0; r < RG; ++r) s += red[part][r][c];
      const size_t o = ((size_t)bh * nb + j) * D + c;
      if (part == 0) {
        const float m = s / (float)cnt;
        kb[c] = m;
        if constexpr (PASS == 0) {
          const __bf16 hi = f2bf(m);
          kbar_hi[o] = hi;
          kbar_lo[o] = f2bf(m - bf2f(hi));
        }
      } else {
        vb[c] = s;
        if constexpr (PASS == 0) vsum[o] = f2bf(s);
      }
    }
    // V^T K over the tile's 64 rows (zero rows past the block add nothing)
#pragma unroll
    for (int ks = 0; ks < kBlock / 16; ++ks) {
      bf16x8 av[NT], bk[NT];
#pragma unroll
      for (int a = 0; a < NT; ++a) av[a] = tr_operand<D, 8, 4>(Vs, 16 * ks, r0 + 32 * a, lane);
#pragma unroll
      for (int b = 0; b < NT; ++b) bk[b] = tr_operand<D, 8, 4>(Ks, 16 * ks, c0 + 32 * b, lane);
#pragma unroll
      for (int a = 0; a < NT; ++a)
#pragma unroll
        for (int b = 0; b < NT; ++b) acc[a][b] = mfma32(av[a], bk[b], acc[a][b]);
    }
    __syncthreads();  // kb, vb published
    // H_j^T = V^T K - vs kbar^T (PASS 0 keeps summing over the chunk's blocks)
    float ss = 0.f;
#pragma unroll
    for (int a = 0; a < NT; ++a)
#pragma unroll
      for (int b = 0; b < NT; ++b) {
        const float kc = kb[c0 + 32 * b + lane % 32];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int c = r0 + 32 * a + 8 * (i / 4) + 4 * g + i % 4;
          acc[a][b][i] = fmaf(-vb[c], kc, acc[a][b][i]);
          if constexpr (PASS == 1) {
            const float dlt = acc[a][b][i] - hb[a][b][i];
            ss = fmaf(dlt, dlt, ss);
          }
        }
        if constexpr (PASS == 1) acc[a][b] = f32x16{};
      }
    if constexpr (PASS == 1) {
      ss = wave_sum(ss);
      if (lane == 0) sqw[wave] = ss;
      __syncthreads();
      if (tid == 0) {
        float t = 0.f;
#pragma unroll
        for (int w = 0; w < kStatThreads / kWave; ++w) t += sqw[w];
        const float m = sqrtf(t);
        Mout[(size_t)bh * nb + j] = m;
        lnM[(size_t)bh * nb + j] = m > 0.f ? logf(m) : -INFINITY;
      }
    }
  }

  if constexpr (PASS == 0) {
    // chunk partial of sum_j H_j^T / n_b in the [c][c'] layout of the state reduction
    float* hp = h_part + ((size_t)bh * gridDim.x + chunk) * D * D;
#pragma unroll
    for (int a = 0; a < NT; ++a)
#pragma unroll
      for (int b = 0; b < NT; ++b)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int c = r0 + 32 * a + 8 * (i / 4) + 4 * g + i % 4;
          const int cp = c0 + 32 * b + lane % 32;
          hp[(size_t)c * D + cp] = acc[a][b][i] * inv_nb;
        }
  }
}

template <class T, int D>
hipError_t launch_pisa_stats_t(const Dims& p, const void* K, const void* V, __bf16* kbar_hi,
                               __bf16* kbar_lo, __bf16* vsum, float* h_part, __bf16* hbar_t,
                               float* hbar, float* M, float* lnM, hipStream_t stream) {
  const int cb = state_chunk_blocks(p);
  dim3 grid((p.nb + cb - 1) / cb, p.B * p.H);
  pisa_stats_kernel<T, D, 0><<<grid, kStatThreads, 0, stream>>>(
      (const T*)K, (const T*)V, p.N, p.nb, cb, kbar_hi, kbar_lo, vsum, h_part, nullptr, nullptr,
      nullptr);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // Hbar^T (bf16) and Hbar (fp32) from the chunk partials; no Z, no low half
  e = launch_state_reduce(p, h_part, nullptr, hbar_t, nullptr, nullptr, hbar, stream);
  if (e != hipSuccess) return e;
  pisa_stats_kernel<T, D, 1><<<grid, kStatThreads, 0, stream>>>(
      (const T*)K, (const T*)V, p.N, p.nb, cb, nullptr, nullptr, nullptr, nullptr, hbar, M, lnM);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_pisa_stats(const Dims& p, const void* K, const void* V, __bf16* kbar_hi,
                             __bf16* kbar_lo, __bf16* vsum, float* h_part, __bf16* hbar_t,
                             float* hbar, float* M, float* lnM, hipStream_t stream) {
  if (p.dtype == kBF16 && p.d == 128)
    return launch_pisa_stats_t<__bf16, 128>(p, K, V, kbar_hi, kbar_lo, vsum, h_part, hbar_t, hbar, M, lnM, stream);
  if (p.dtype == kBF16 && p.d == 64)
    return launch_pisa_stats_t<__bf16, 64>(p, K, V, kbar_hi, kbar_lo, vsum, h_part, hbar_t, hbar, M, lnM, stream);
  if (p.dtype == kF32 && p.d == 128)
    return launch_pisa_stats_t<float, 128>(p, K, V, kbar_hi, kbar_lo, vsum, h_part, hbar_t, hbar, M, lnM, stream);
  return launch_pisa_stats_t<float, 64>(p, K, V, kbar_hi, kbar_lo, vsum, h_part, hbar_t, hbar, M, lnM, stream);
}

}  // namespace sla
