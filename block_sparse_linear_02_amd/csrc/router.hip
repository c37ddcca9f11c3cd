// router.hip - the SLA2 router on gfx950 (SLA2 Italian summary section 2.B, Arabic summary
// sections 2.ba and 2.dal): block mean-pool of Q and K, learnable projections, block-score map
// and the inference-time HardTop-k.
//
//   pool_project_kernel  one workgroup per (8 blocks, head, Q|K): streams the blocks' rows
//                        (16-byte coalesced loads, two blocks in flight, fp32 sums reduced
//                        inside each wavefront by shuffles, per-wavefront partials in LDS and
//                        one barrier after the last block), divides by the number of valid
//                        tokens, multiplies by W (fp32) and stores the result split into a
//                        bf16 high part and a bf16 low part (x = hi + lo + O(2^-17 |x|)).
//   score_topk_kernel    one workgroup per (16 query blocks, head), each XCD taking a
//                        contiguous range of heads: the 16 x n_b score tile
//                        s = (q~ . k~) / sqrt(d) by bf16 MFMA on the split operands
//                        (hi*hi + hi*lo + lo*hi, fp32 accumulation: about fp32 accuracy) into
//                        LDS (8 wavefronts, each key tile's operands loaded through a range-
//                        checked buffer resource while the previous tile's MFMAs run), then per
//                        row (one wavefront) the k-th largest score by a bitwise search on
//                        order-preserving keys (counts by ballot): the top 12 bits over every
//                        key, the low 20 over the band of keys sharing those bits, compacted in
//                        LDS; then an ascending compaction that keeps the lowest indices among
//                        equal scores.
#include "sla_device.hpp"
#include "sla_launch.hpp"
#include "sla_tiles.hpp"

namespace sla {

namespace {

constexpr int kPoolBlocksPerWg = 8;
constexpr int kPoolDepth = 2;  // blocks whose loads a thread keeps in flight
constexpr int kPoolThreads = 256;

// element v of a 16-byte load of T values, as float
template <class T>
__device__ __forceinline__ float raw_elem(i32x4 x, int v);
template <>
__device__ __forceinline__ float raw_elem<__bf16>(i32x4 x, int v) {
  const u32 w = (u32)x[v / 2];
  return __uint_as_float(v % 2 ? (w & 0xffff0000u) : (w << 16));
}
template <>
__device__ __forceinline__ float raw_elem<float>(i32x4 x, int v) { return __int_as_float(x[v]); }

template <class T, int D>
__global__ __launch_bounds__(kPoolThreads) void pool_project_kernel(
    const T* __restrict__ Q, const T* __restrict__ K, const float* __restrict__ Wq,
    const float* __restrict__ Wk, int N, int nb, __bf16* __restrict__ q_hi,
    __bf16* __restrict__ q_lo, __bf16* __restrict__ k_hi, __bf16* __restrict__ k_lo) {
  constexpr int VEC = 16 / sizeof(T);      // elements per 16-byte load
  constexpr int TPR = D / VEC;             // threads per row
  constexpr int RPP = kPoolThreads / TPR;  // rows per pass
  constexpr int NW = kPoolThreads / kWave;
  static_assert(kBlock % RPP == 0, "rows per pass must divide the block");
  static_assert(TPR <= kWave && kWave % TPR == 0, "a row is read by lanes of one wavefront");
  __shared__ float part[kPoolBlocksPerWg][NW][D];  // per-wavefront column sums of each block
  __shared__ float xbar[kPoolBlocksPerWg][D];

  const int tid = threadIdx.x;
  const int lane = tid % kWave;
  const int wave = tid / kWave;
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

  // block b's rows as raw 16-byte loads: every load issued unconditionally (rows past N re-read
  // the block's last row and are dropped in the sum; a block past n_b re-reads the last block),
  // and block b + kPoolDepth - 1's loads go out before block b's sum, so each thread keeps
  // kPoolDepth blocks' loads in flight.  A block's column sums are reduced inside each wavefront (the lanes reading the
  // same columns, by shuffles) and left per wavefront in LDS: no barrier until every block is
  // summed.
  i32x4 tmp[kPoolDepth][kBlock / RPP];
  auto load_block = [&](int b, i32x4 (&dst)[kBlock / RPP]) {
    const int row0 = min(t0 + b, nb - 1) * kBlock;
    const int last = min(kBlock, N - row0) - 1;
#pragma unroll
    for (int p = 0; p < kBlock / RPP; ++p) dst[p] = ld16(X + (size_t)(row0 + min(roff + p * RPP, last)) * D + col);
  };
#pragma unroll
  for (int b = 0; b + 1 < kPoolDepth; ++b) load_block(b, tmp[b]);
#pragma unroll
  for (int b = 0; b < kPoolBlocksPerWg; ++b) {
    if (b + kPoolDepth - 1 < kPoolBlocksPerWg)
      load_block(b + kPoolDepth - 1, tmp[(b + kPoolDepth - 1) % kPoolDepth]);
    if (b < nblk) {
      const int cnt = min(kBlock, N - (t0 + b) * kBlock);
      float acc[VEC];
#pragma unroll
      for (int v = 0; v < VEC; ++v) acc[v] = 0.f;
#pragma unroll
      for (int p = 0; p < kBlock / RPP; ++p)
#pragma unroll
        for (int v = 0; v < VEC; ++v) acc[v] += roff + p * RPP < cnt ? raw_elem<T>(tmp[b % kPoolDepth][p], v) : 0.f;
#pragma unroll
      for (int o = TPR; o < kWave; o <<= 1)
#pragma unroll
        for (int v = 0; v < VEC; ++v) acc[v] += __shfl_xor(acc[v], o);
      if (lane < TPR) {
#pragma unroll
        for (int v = 0; v < VEC; ++v) part[b][wave][col + v] = acc[v];
      }
    }
  }
  __syncthreads();
  for (int e = tid; e < nblk * D; e += kPoolThreads) {
    const int b = e / D, c = e % D;
    float sum = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) sum += part[b][w][c];
    xbar[b][c] = sum / (float)min(kBlock, N - (t0 + b) * kBlock);
  }
  __syncthreads();

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
// the float whose order-preserving key (float_key) is 0, below the key of every score: the
// all-ones bit pattern (a NaN, never produced by the score arithmetic on finite inputs)
#define kKeyZero __uint_as_float(0xffffffffu)

// score row pitch in floats: a multiple of 16 plus 4, so that the four rows one MFMA result
// register spans (4 apart) start 16 banks apart and a score store is free of bank conflicts
__host__ __device__ constexpr int score_pitch(int nb) { return (nb + 15) / 16 * 16 + 4; }

// Scores of 16 query blocks against all key blocks into LDS, then per row the k-th largest
// score and the ascending compaction.  NCH = key slots per lane (at least ceil(n_b / 64)):
// slots past n_b hold key 0, below every valid key.  bias (optional, [bh][n_b]) is added to
// every score of key block j before the selection; probs receives the row softmax of the
// scores, or (raw) the scores themselves.
template <int D, int NCH>
__global__ __launch_bounds__(kTopkThreads) void score_topk_kernel(
    const __bf16* __restrict__ q_hi, const __bf16* __restrict__ q_lo,
    const __bf16* __restrict__ k_hi, const __bf16* __restrict__ k_lo, int nb, int topk,
    float scale, int nbp, const float* __restrict__ bias, int raw, int32_t* __restrict__ idx,
    uint8_t* __restrict__ mask, float* __restrict__ probs) {
  extern __shared__ float S[];  // [kRowsPerWg][nbp]
  const int lane = threadIdx.x % kWave;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);  // wavefront-uniform
  // workgroup -> (head, 16-row tile): each XCD takes a contiguous range of the head-major
  // items, so the workgroups sharing a head's key projections share that XCD's L2
  const int ntile_rows = (nb + kRowsPerWg - 1) / kRowsPerWg;
  const int item = xcd_remap(blockIdx.x, (int)gridDim.x);  // gridDim.x = row tiles x heads
  const int bh = item / ntile_rows;
  const int i0 = (item % ntile_rows) * kRowsPerWg;
  const size_t base = (size_t)bh * nb * D;

  // ---- scores: 16 x n_b tile, 16x16x32 MFMA on split operands (hi*hi + hi*lo + lo*hi) ----
  // Operands come through buffer resources over the head's projections: rows past n_b read
  // zero (range check), so no load sits behind a branch.  Wavefront w takes the key tiles
  // w, w + 8, ..., each tile's loads issued while the previous tile's MFMAs run.
  {
    constexpr int KS = D / 32;
    const uint32_t bytes = (uint32_t)((size_t)nb * D * sizeof(__bf16));
    const __amdgpu_buffer_rsrc_t rqh = make_rsrc(q_hi + base, bytes), rql = make_rsrc(q_lo + base, bytes);
    const __amdgpu_buffer_rsrc_t rkh = make_rsrc(k_hi + base, bytes), rkl = make_rsrc(k_lo + base, bytes);
    // lane's row of a 16-row tile and its 8 columns of k step s: (lane % 16, 32 s + 8 (lane / 16))
    const uint32_t loff = (uint32_t)(((lane % 16) * D + 8 * (lane / 16)) * sizeof(__bf16));
    auto ld = [&](__amdgpu_buffer_rsrc_t r, uint32_t off) -> bf16x8 {
      return __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0));
    };
    bf16x8 ahi[KS], alo[KS];
    const uint32_t aoff = loff + (uint32_t)(i0 * D * sizeof(__bf16));
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      ahi[s] = ld(rqh, aoff + 64 * s);
      alo[s] = ld(rql, aoff + 64 * s);
    }
    const int ntiles = (nb + 15) / 16;
    bf16x8 bhi[2][KS], blo[2][KS];
    auto load_tile = [&](int t, bf16x8 (&h)[KS], bf16x8 (&l)[KS]) {
      const uint32_t off = loff + (uint32_t)(t * 16 * D * sizeof(__bf16));
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        h[s] = ld(rkh, off + 64 * s);
        l[s] = ld(rkl, off + 64 * s);
      }
    };
    auto score_tile = [&](int t, const bf16x8 (&h)[KS], const bf16x8 (&l)[KS]) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        acc = mfma16(alo[s], h[s], acc);
        acc = mfma16(ahi[s], l[s], acc);
        acc = mfma16(ahi[s], h[s], acc);
      }
      const int j = t * 16 + lane % 16;  // columns past n_b land in the row padding
      const bool jok = j < nb;
      const float bj = (bias && jok) ? bias[(size_t)bh * nb + j] : 0.f;
#pragma unroll
      for (int r = 0; r < 4; ++r)
        S[(4 * (lane / 16) + r) * nbp + j] = jok ? fmaf(acc[r], scale, bj) : kKeyZero;
    };
    // the row padding past the last 16-column tile
    for (int e = threadIdx.x; e < kRowsPerWg * (nbp - 16 * ntiles); e += kTopkThreads)
      S[(e / (nbp - 16 * ntiles)) * nbp + 16 * ntiles + e % (nbp - 16 * ntiles)] = kKeyZero;
    // tiles past the last one read zero (range check) and are never scored
    load_tile(wave, bhi[0], blo[0]);
    for (int t = wave; t < ntiles; t += 2 * kTopkWaves) {
      load_tile(t + kTopkWaves, bhi[1], blo[1]);
      score_tile(t, bhi[0], blo[0]);
      if (t + kTopkWaves >= ntiles) break;
      load_tile(t + 2 * kTopkWaves, bhi[0], blo[0]);
      score_tile(t + kTopkWaves, bhi[1], blo[1]);
    }
  }
  __syncthreads();

  // ---- per row: the k-th largest key T, then ascending compaction ----
  // T is found bit by bit from the top: T is the largest value with at least topk keys >= T, so
  // bit b of T is set iff count(key >= T | 2^b) >= topk, a count taken by ballots.  After the
  // top 12 bits the k-th largest key lies in the band of keys sharing T's top 12 bits (a band
  // an eighth of a binade wide, which typically holds a few percent of the scores); the keys
  // above the band are counted, the band's keys are compacted into the row's LDS storage (the
  // scores are in registers by then), and the low 20 bits are searched over the band alone
  // (two keys per lane).  A band of more than 128 keys (many equal scores) keeps the search over
  // every key.  The padding columns of a score row hold the float whose key is 0 (below every
  // score), so the slots past n_b need no test.
  // The lane index is laundered through an empty asm in every row so that the compiler keeps
  // no per-lane comparison across rows (it would hold them as scalar masks and spill them).
  constexpr int kBandShift = 20;
  for (int r = wave; r < kRowsPerWg; r += kTopkWaves) {
    const int i = i0 + r;
    if (i >= nb) break;
    int ln = lane;
    asm volatile("" : "+v"(ln));
    const uint64_t lt_mask = (ln == 0) ? 0ull : (~0ull >> (64 - ln));
    float* srow = S + r * nbp;
    if (probs && raw) {
      float* prow = probs + ((size_t)bh * nb + i) * nb;
      for (int j = ln; j < nb; j += kWave) prow[j] = srow[j];
    } else if (probs) {
      float mx = -INFINITY;
      for (int j = ln; j < nb; j += kWave) mx = fmaxf(mx, srow[j]);
      mx = wave_max(mx);
      float sum = 0.f;
      for (int j = ln; j < nb; j += kWave) sum += __expf(srow[j] - mx);
      sum = wave_sum(sum);
      const float inv = 1.f / sum;
      float* prow = probs + ((size_t)bh * nb + i) * nb;
      for (int j = ln; j < nb; j += kWave) prow[j] = __expf(srow[j] - mx) * inv;
    }
    u32 key[NCH];
#pragma unroll
    for (int c = 0; c < NCH; ++c) key[c] = float_key(srow[min(c * kWave + ln, nbp - 1)]);
    u32 T = 0xffffffffu;  // topk == 0: nothing is kept
    if (topk > 0) {
      T = 0;
      for (int bit = 31; bit >= kBandShift; --bit) {
        const u32 cand = T | (1u << bit);
        int cnt = 0;
#pragma unroll
        for (int c = 0; c < NCH; ++c) cnt += __popcll(__ballot(key[c] >= cand));
        if (cnt >= topk) T = cand;
      }
      const u32 tb = T >> kBandShift;
      int above = 0, m = 0;
      u32* band = reinterpret_cast<u32*>(srow);
      __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");  // the score reads come first
      __builtin_amdgcn_wave_barrier();
#pragma unroll
      for (int c = 0; c < NCH; ++c) {
        above += __popcll(__ballot((key[c] >> kBandShift) > tb));
        const bool inb = (key[c] >> kBandShift) == tb && key[c] != 0u;
        const uint64_t bmask = __ballot(inb);
        const int at = m + __popcll(bmask & lt_mask);
        if (inb && at < nbp) band[at] = key[c];
        m += __popcll(bmask);
      }
      __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
      __builtin_amdgcn_wave_barrier();
      if (m <= 2 * kWave) {
        const int need = topk - above;  // 1 <= need <= m
        const u32 b0 = ln < m ? band[ln] : 0u;
        const u32 b1 = ln + kWave < m ? band[ln + kWave] : 0u;
        for (int bit = kBandShift - 1; bit >= 0; --bit) {
          const u32 cand = T | (1u << bit);
          const int cnt = __popcll(__ballot(b0 >= cand)) + __popcll(__ballot(b1 >= cand));
          if (cnt >= need) T = cand;
        }
      } else {
        for (int bit = kBandShift - 1; bit >= 0; --bit) {
          const u32 cand = T | (1u << bit);
          int cnt = 0;
#pragma unroll
          for (int c = 0; c < NCH; ++c) cnt += __popcll(__ballot(key[c] >= cand));
          if (cnt >= topk) T = cand;
        }
      }
    }
    int32_t* irow = idx + ((size_t)bh * nb + i) * topk;
    uint8_t* mrow = mask ? mask + ((size_t)bh * nb + i) * nb : nullptr;
    if (topk > 0) {
      int gt = 0;
#pragma unroll
      for (int c = 0; c < NCH; ++c) gt += __popcll(__ballot(key[c] > T));
      const int need = topk - gt;  // equal keys to keep, lowest index first
      int pos = 0, ties = 0;
#pragma unroll
      for (int c = 0; c < NCH; ++c) {
        const int j = c * kWave + ln;
        const bool eq = key[c] == T;  // T >= 1, so no slot past n_b is equal or above
        const uint64_t eqm = __ballot(eq);
        const int rank = ties + __popcll(eqm & lt_mask);
        const bool sel = key[c] > T || (eq && rank < need);
        const uint64_t selm = __ballot(sel);
        const int at = pos + __popcll(selm & lt_mask);
        if (sel && at < topk) irow[at] = j;  // at < topk always; the test keeps idx in bounds
        if (mrow && j < nb) mrow[j] = sel ? 1 : 0;
        pos += __popcll(selm);
        ties += __popcll(eqm);
      }
    } else if (mrow) {
      for (int j = ln; j < nb; j += kWave) mrow[j] = 0;
    }
  }
}

template <int D>
hipError_t launch_topk(const Dims& p, const __bf16* q_hi, const __bf16* q_lo,
                       const __bf16* k_hi, const __bf16* k_lo, const float* bias, int raw,
                       int32_t* idx, uint8_t* mask, float* probs, size_t lds,
                       hipStream_t stream) {
  const int nbp = score_pitch(p.nb);
  // a 1-D grid: one workgroup per (16-row tile, head)
  dim3 grid((p.nb + kRowsPerWg - 1) / kRowsPerWg * p.B * p.H, 1);
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
  return (size_t)kRowsPerWg * score_pitch(nb) * sizeof(float);
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
