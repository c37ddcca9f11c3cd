// sparse_split.hip - block-sparse softmax branch and alpha combine on gfx950, with the linear
// branch's per-query-block state T_i = H - sum_{j in sel(i)} h_j taken from memory (formed for
// every query block at once by the mask-product kernel, linear_gemm.hip).
//
// Sources: SLA2 Italian summary sections 1 and 2.A and Arabic summary sections 1 and 2.alef
// (sparse branch renormalised over the kept blocks; O = alpha O_s + (1 - alpha) O_l); SALAD
// section 2 (ReLU feature map of the linear branch, over the blocks the sparse branch leaves).
//
// One workgroup = one query block (64 rows) of one (batch, head), four wavefronts doing the same
// work on different quarters, split over keys: wavefront w = 2 kh + qh takes query rows
// 32 qh .. 32 qh + 31 against keys 32 kh .. 32 kh + 31 of every kept tile.  S^T = K Q^T
// (v_mfma_f32_32x32x16_bf16; each lane owns one query row, so the row statistics stay in-lane),
// online softmax in the log2 domain with a lazy rescale (the running maximum only moves when a
// row's maximum grows by more than 2^8), P rounded to bf16, row sums from the bf16 P with
// v_dot2, O_s^T += V^T P^T with V read transposed from LDS (ds_read_b64_tr_b16).  The two key
// halves of a row are merged once at the end (max / rescale / add of two partial softmax
// states).  K_j, V_j tiles are double-buffered in LDS, one array per buffer so that the compiler
// can tell the buffer being filled by direct-to-LDS loads from the one being read.
// Epilogue: T_i^T (bf16, [c][c']) is loaded into a free tile buffer, zeta = Z -
// sum_kept z_j; wavefront (qh, kh) computes, for its 32 rows and channel half kh,
// num = relu(Q) T_i by MFMA, den = relu(q) . zeta, and O = alpha O_s / l + (1 - alpha) num / den
// (the linear part is 0 when nothing is unselected or den == 0), fp32 stores; rows past N are
// not stored.
#include <type_traits>

#include "sla_device.hpp"
#include "sla_launch.hpp"
#include "sla_tiles.hpp"

namespace sla {

namespace {

constexpr int kSplitThreads = 256;

template <class T>
__device__ __forceinline__ bf16x8 load_row8(const T* p);
template <>
__device__ __forceinline__ bf16x8 load_row8<__bf16>(const __bf16* p) {
  return *reinterpret_cast<const bf16x8*>(p);
}
template <>
__device__ __forceinline__ bf16x8 load_row8<float>(const float* p) {
  const f32x4 a = *reinterpret_cast<const f32x4*>(p);
  const f32x4 b = *reinterpret_cast<const f32x4*>(p + 4);
  return bf16x8{f2bf(a[0]), f2bf(a[1]), f2bf(a[2]), f2bf(a[3]),
                f2bf(b[0]), f2bf(b[1]), f2bf(b[2]), f2bf(b[3])};
}

// fp32 inputs: the bf16 remainder x - bf16(x) of 8 consecutive values (0 for bf16 inputs)
template <class T>
__device__ __forceinline__ bf16x8 load_row8_lo(const T* p) {
  if constexpr (sizeof(T) == 2) {
    return bf16x8{};
  } else {
    const f32x4 a = *reinterpret_cast<const f32x4*>(p);
    const f32x4 b = *reinterpret_cast<const f32x4*>(p + 4);
    bf16x8 r;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      r[e] = f2bf(a[e] - bf2f(f2bf(a[e])));
      r[e + 4] = f2bf(b[e] - bf2f(f2bf(b[e])));
    }
    return r;
  }
}

// sum of the 8 bf16 values of v (fp32 accumulation)
__device__ __forceinline__ float sum8(bf16x8 v, float acc) {
  const bf16x2 one = {f2bf(1.f), f2bf(1.f)};
#pragma unroll
  for (int i = 0; i < 4; ++i) acc = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{v[2 * i], v[2 * i + 1]}, one, acc, false);
  return acc;
}

constexpr float kRescaleSlack = 8.f;  // log2 units: P may reach 2^8 before the maximum moves

// Compile-time shape of the kernel's LDS use and MFMA tiling.
template <class T, int D>
struct SplitShape {
  static constexpr int NS = D / 16;       // MFMA k-steps over the head dim
  static constexpr int NC = D / 32;       // 32-channel tiles of O
  static constexpr int HC = NC / 2;       // 32-wide tiles in half of the head dim
  static constexpr int PITCH = D + kPad;  // row pitch of the epilogue's T^T array (bf16 elements)
  static constexpr int TILE = TileLayout<D>::ELEMS;
  // fp32 inputs keep K as bf16 hi + lo tiles so that S = K Q^T is about fp32-accurate
  // (Kh Qh + Kh Ql + Kl Qh); bf16 inputs are exact in one bf16 tile
  static constexpr bool SPLIT = sizeof(T) == 4;
  static constexpr int TILES = SPLIT ? 3 : 2;  // per buffer: K (hi), V, [K lo]
  // LDS: three separate arrays (bf16 elements), so that the compiler can tell the buffer being
  // filled by direct-to-LDS loads from the one being read and does not wait for the former
  // before reading the latter:
  //   QBUF: the Q tile(s) (hi [, lo]); after the loop, zeta and the exchanged row statistics;
  //   BUF (x2): one K/V tile set each; after the loop, the split-K exchange, then T^T hi (buffer
  //   0) and lo (buffer 1), each [D][D] in the tile row layout.
  static constexpr int QTILES = SPLIT ? 2 : 1;
  static constexpr int QBUF = QTILES * TILE;
  static constexpr int BUF = TILES * TILE;
  static constexpr int MERGE = 4 * HC * 16 * kWave * 2;
  static_assert(MERGE <= BUF, "split-K exchange must fit in one tile buffer");
  static_assert(D * TileLayout<D>::PITCH <= BUF, "T^T must fit in one tile buffer");
  static_assert(2 * D + 2 * 4 * 2 * 32 <= QBUF, "epilogue scalars must fit in the Q buffer");
};

template <class T, int D, int QH, int KH>
__device__ __forceinline__ void split_wave(
    const T* __restrict__ Q, const T* __restrict__ K, const T* __restrict__ V,
    const int32_t* __restrict__ idx, const float* __restrict__ alpha,
    const __bf16* __restrict__ t_g, const float* __restrict__ Z, const float* __restrict__ zb,
    float* __restrict__ O, int N, int nb, int topk, float c_log2, __bf16* lq, __bf16* lb0,
    __bf16* lb1, int bh, int qb) {
  using S_ = SplitShape<T, D>;
  constexpr int NS = S_::NS, NC = S_::NC, HC = S_::HC, PITCH = S_::PITCH, TILE = S_::TILE;
  constexpr bool SPLIT = S_::SPLIT;
  constexpr int TILES = S_::TILES;
  float* zeta = reinterpret_cast<float*>(lq);        // [D]
  float* ml = reinterpret_cast<float*>(lq + 2 * D);  // [4 wavefronts][max, sum][32 rows]
  // the tile buffer of a compile-time index
  auto buf = [&](auto BUFC) -> __bf16* { return decltype(BUFC)::value ? lb1 : lb0; };
  constexpr int qh = QH, kh = KH, w = 2 * KH + QH;
  const int tid = threadIdx.x;
  const int lane = tid % kWave, g = lane / 32;
  const size_t hoff = (size_t)bh * N * D;
  const int32_t* sel = idx + ((size_t)bh * nb + qb) * topk;

  // Tile staging: every thread moves its share of each tile.  bf16 tiles with d = 128 and all
  // 64 rows valid go HBM -> LDS directly (no registers), issued at the start of the iteration
  // that uses the other buffer; other tiles (fp32 inputs, d = 64, the short last block) go
  // through registers with zero fill, stored right away.  z_j travels with the tile.
  constexpr bool DIRECT = sizeof(T) == 2 && D == 128;
  const bool z_lane = tid < D;
  float z_in = 0.f;      // z_j of the tile being staged
  int nv_next = kBlock;  // valid rows of the tile being staged
  float zacc = 0.f;      // sum of z_j over the staged kept blocks (threads tid < D)
  // DIRECT tiles with fewer than 64 valid rows: zero the tail once every load has landed and
  // been published by a barrier (wavefront-uniform condition; at most once per head)
  auto zero_tail = [&](auto BUFC, int nv) {
    if constexpr (DIRECT) {
      if (nv < kBlock) {
        __bf16* dst = buf(BUFC);
        zero_tile_rows<kSplitThreads>(dst, tid, nv);
        zero_tile_rows<kSplitThreads>(dst + TILE, tid, nv);
        __syncthreads();
      }
    }
  };
  auto stage = [&](int t, auto BUFC) {
    const int j = sel[t];
    const int nv = min(kBlock, N - j * kBlock);
    __bf16* dst = buf(BUFC);
    const T* ksrc = K + hoff + (size_t)j * kBlock * D;
    const T* vsrc = V + hoff + (size_t)j * kBlock * D;
    if (z_lane) z_in = zb[((size_t)bh * nb + j) * D + tid];
    nv_next = nv;
    if constexpr (DIRECT) {
      // a short tile (the last block of the sequence) is clamped here and its tail rows are
      // zeroed after the loads land (zero_tail), so no register path sits in the loop
      if (nv == kBlock) {
        load_tile_direct<kSplitThreads>(ksrc, dst, tid);
        load_tile_direct<kSplitThreads>(vsrc, dst + TILE, tid);
      } else {
        load_tile_direct_clamped<kSplitThreads>(ksrc, dst, tid, nv);
        load_tile_direct_clamped<kSplitThreads>(vsrc, dst + TILE, tid, nv);
      }
    } else {
      TileLoader<T, D, kSplitThreads> lk, lv;
      lk.load(ksrc, nv, tid);
      lv.load(vsrc, nv, tid);
      if constexpr (SPLIT)
        lk.store_split(dst, dst + 2 * TILE, tid);
      else
        lk.store(dst, tid);
      lv.store(dst + TILE, tid);
    }
  };

  // Q tile of the query block (rows past N zero-filled), staged once into LDS in the K tile
  // layout; the B operand of S^T = K Q^T is re-read from there each tile (k-slot 8g + jj of step
  // s <-> channel 16s + 8g + jj), which keeps 32 registers per lane free for the accumulators
  const int m = 32 * qh + lane % 32;
  const int row = qb * kBlock + m;
  const bool row_ok = row < N;
  {
    const int nq = min(kBlock, N - qb * kBlock);
    const T* qsrc = Q + hoff + (size_t)qb * kBlock * D;
    if (DIRECT && nq == kBlock) {
      if constexpr (DIRECT) load_tile_direct<kSplitThreads>(qsrc, lq, tid);
    } else {
      TileLoader<T, D, kSplitThreads> lqt;
      lqt.load(qsrc, nq, tid);
      if constexpr (SPLIT)
        lqt.store_split(lq, lq + TILE, tid);
      else
        lqt.store(lq, tid);
    }
  }
  const __bf16* Qs = lq;
  f32x16 os[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) os[c] = f32x16{};
  float mrun = -INFINITY, lsum = 0.f;
  constexpr int c0 = kh * (D / 2);  // this wavefront's output channel half
  // LDS operand reads.  d = 128: per-lane address parts computed once and laundered through an
  // empty asm at the start of every tile (so the compiler re-derives the per-block addresses
  // with one v_xor each instead of hoisting dozens of them into registers); row and tile
  // offsets are immediates.  d = 64: the padded layout's plain offsets.
  constexpr bool XADDR = D == 128;
  int ap_row = 0, ap_va = 0, ap_vb = 0, ap_sa = 0, ap_sb = 0;
  if constexpr (XADDR) {
    ap_row = row_part(lane);
    ap_va = tr_part<4>(lane, 0);
    ap_vb = tr_part<4>(lane, 8);
    ap_sa = tr_part<8>(lane, 0);
    ap_sb = tr_part<8>(lane, 4);
  }
  auto launder = [&]() {
    if constexpr (XADDR) asm volatile("" : "+v"(ap_row), "+v"(ap_va), "+v"(ap_vb), "+v"(ap_sa), "+v"(ap_sb));
  };
  // row-wise operand: row R0 + lane%32 (R0 % 32 == 0), channels 16k + 8g .. + 7
  auto rd_row = [&](const __bf16* tile, int R0, int k) -> bf16x8 {
    if constexpr (XADDR)
      return lds_row16(tile, R0 * 256 + (ap_row ^ (32 * k)));
    else
      return *reinterpret_cast<const bf16x8*>(tile + TileLayout<D>::off(R0 + lane % 32, 16 * k + 8 * g));
  };
  // transposed operands (tr_operand): PV key order (step 4, gap 8) and state order (8, 4)
  auto rd_tr_v = [&](const __bf16* tile, int row0, int col0) -> bf16x8 {
    if constexpr (XADDR)
      return join_tr(lds_tr_at(tile, row0 * 256 + (ap_va ^ (2 * col0))),
                     lds_tr_at(tile, row0 * 256 + (ap_vb ^ (2 * col0))));
    else
      return tr_operand<D, 4, 8>(tile, row0, col0, lane);
  };
  auto rd_tr_s = [&](const __bf16* tile, int row0, int col0) -> bf16x8 {
    if constexpr (XADDR)
      return join_tr(lds_tr_at(tile, row0 * 256 + (ap_sa ^ (2 * col0))),
                     lds_tr_at(tile, row0 * 256 + (ap_sb ^ (2 * col0))));
    else
      return tr_operand<D, 8, 4>(tile, row0, col0, lane);
  };

  int nv_cur = kBlock;
  if (topk > 0) {
    stage(0, std::integral_constant<int, 0>{});
    zacc += z_in;
    nv_cur = nv_next;
    wait_vmem();
    __syncthreads();
    zero_tail(std::integral_constant<int, 0>{}, nv_cur);
  }
  // one kept tile; BUF (= t & 1, a compile-time constant through the unrolled pair below) is
  // the buffer holding tile t, and tile t + 1 is staged into the other one (last read in
  // iteration t - 1)
  auto step = [&](int t, auto BUFC) {
    constexpr int BUF = decltype(BUFC)::value;
    const int nv = nv_cur;
    launder();
    if (t + 1 < topk) stage(t + 1, std::integral_constant<int, 1 - BUF>{});
    const __bf16* Ks = buf(BUFC);
    const __bf16* Vs = Ks + TILE;
    if (nv > 32 * kh) {  // this wavefront's key half holds valid keys (wavefront-uniform)
      // S^T for keys 32kh + lane%32
      // operands in groups of four k-steps (the scheduling barriers keep the compiler from
      // hoisting every LDS read of the tile at once, which would exhaust the registers)
      bf16x8 ka[NS], qa[NS];
      f32x16 s = f32x16{};
#pragma unroll
      for (int k = 0; k < NS; ++k) {
        if (k % 4 == 0) {
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int kk = k; kk < k + 4 && kk < NS; ++kk) {
            ka[kk] = rd_row(Ks, 32 * kh, kk);
            qa[kk] = rd_row(Qs, 32 * qh, kk);
          }
        }
        if constexpr (SPLIT) {
          const bf16x8 ql = rd_row(Qs + TILE, 32 * qh, k);
          s = mfma32(rd_row(Ks + 2 * TILE, 32 * kh, k), qa[k], s);
          s = mfma32(ka[k], ql, s);
        }
        s = mfma32(ka[k], qa[k], s);
      }
      __builtin_amdgcn_sched_barrier(0);
      // key of accumulator register i: 32kh + 8(i/4) + 4g + i%4
      if (nv < 32 * kh + 32) {
        const int lim = nv - (32 * kh + 4 * g);
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (8 * (i / 4) + i % 4 >= lim) s[i] = -INFINITY;
      }
      float mx = s[0];
#pragma unroll
      for (int i = 1; i < 16; ++i) mx = fmaxf(mx, s[i]);
      mx = xor32_max(mx) * c_log2;
      if (__ballot(mx > mrun + kRescaleSlack)) {
        const float mnew = fmaxf(mrun, mx);
        const float corr = fast_exp2(mrun - mnew);
        mrun = mnew;
        lsum *= corr;
#pragma unroll
        for (int c = 0; c < NC; ++c) os[c] *= corr;
      }
      bf16x8 pb[2];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) pb[u][jj] = f2bf(fast_exp2(fmaf(s[8 * u + jj], c_log2, -mrun)));
        lsum = sum8(pb[u], lsum);
      }
      // O^T += V^T P^T ; MFMA u covers the keys of accumulator registers 8u .. 8u + 7, whose
      // V operand rows are 32kh + 16u + 4g + {0..3, 8..11}; two channel tiles per group
#pragma unroll
      for (int c = 0; c < NC; c += 2) {
        __builtin_amdgcn_sched_barrier(0);
        bf16x8 va[2][2];
#pragma unroll
        for (int cc = 0; cc < 2; ++cc)
#pragma unroll
          for (int u = 0; u < 2; ++u) va[cc][u] = rd_tr_v(Vs, 32 * kh + 16 * u, 32 * (c + cc));
#pragma unroll
        for (int cc = 0; cc < 2; ++cc)
#pragma unroll
          for (int u = 0; u < 2; ++u) os[c + cc] = mfma32(va[cc][u], pb[u], os[c + cc]);
      }
    }
    if (t + 1 < topk) zacc += z_in;
    nv_cur = nv_next;
    wait_vmem();
    __syncthreads();
    if (t + 1 < topk) zero_tail(std::integral_constant<int, 1 - BUF>{}, nv_cur);
  };
  for (int t = 0; t < topk; t += 2) {
    step(t, std::integral_constant<int, 0>{});
    if (t + 1 < topk) step(t + 1, std::integral_constant<int, 1>{});
  }

  // T_i^T [c][c'] into tile buffer 1, free since the last step's barrier (buffer 0 takes the
  // split-K exchange below), in the tile row layout; awaited before the epilogue's MFMAs
  {
    const __bf16* th = t_g + ((size_t)bh * nb + qb) * D * D;
#pragma unroll
    for (int half = 0; half < D / kBlock; ++half) {
      if constexpr (D == 128) {
        load_tile_direct<kSplitThreads>(th + half * kBlock * D, lb1 + half * kBlock * D, tid);
      } else {
        TileLoader<__bf16, D, kSplitThreads> ld;
        ld.load(th + half * kBlock * D, kBlock, tid);
        ld.store(lb1 + half * TILE, tid);
      }
    }
  }

  // ---- merge the two key halves of each row: wavefront w hands the channel half it does not
  // own to its partner w ^ 2 and takes the partner's share of its own half ----
  if (topk == 0) {  // the Q tile's direct loads may still be landing in the region reused below
    wait_vmem();
    __syncthreads();
  }
  lsum = xor32_sum(lsum);
  float* xo = reinterpret_cast<float*>(lb0);  // [wavefront][tile][register][lane]
#pragma unroll
  for (int cc = 0; cc < HC; ++cc)
#pragma unroll
    for (int i = 0; i < 16; ++i) xo[((w * HC + cc) * 16 + i) * kWave + lane] = os[(1 - kh) * HC + cc][i];
  if (g == 0) {
    ml[(w * 2 + 0) * 32 + lane] = mrun;
    ml[(w * 2 + 1) * 32 + lane] = lsum;
  }
  __syncthreads();
  f32x16 oo[HC];  // O_s^T of this wavefront's channel half, both key halves merged
  {
    constexpr int pw = w ^ 2;
    const float mb = ml[(pw * 2 + 0) * 32 + lane % 32], lb = ml[(pw * 2 + 1) * 32 + lane % 32];
    const float mt = fmaxf(mrun, mb);
    const float fa = mrun == -INFINITY ? 0.f : fast_exp2(mrun - mt);
    const float fb = mb == -INFINITY ? 0.f : fast_exp2(mb - mt);
    lsum = lsum * fa + lb * fb;
#pragma unroll
    for (int cc = 0; cc < HC; ++cc)
#pragma unroll
      for (int i = 0; i < 16; ++i)
        oo[cc][i] = os[kh * HC + cc][i] * fa + xo[((pw * HC + cc) * 16 + i) * kWave + lane] * fb;
  }
  const float inv_l = topk > 0 ? 1.f / lsum : 0.f;

  f32x16 num[HC];
  float inv_den = 0.f;
  {
    // this row of Q for the numerator, in flight with the T_i loads (unconditional, from a
    // clamped row: a load under a branch makes the compiler wait for it on the spot)
    bf16x8 qv[NS];
    {
      const T* qr = Q + hoff + (size_t)min(row, N - 1) * D + 8 * g;
#pragma unroll
      for (int k = 0; k < NS; ++k) qv[k] = load_row8<T>(qr + 16 * k);
    }
    if (z_lane) zeta[tid] = Z[(size_t)bh * D + tid] - zacc;
    wait_vmem();
    __syncthreads();
    launder();
    // num^T[c][m] = sum_c' T_i^T[c][c'] relu(Q)[m][c'] over this wavefront's channel half: the
    // A operand (rows c, k = c') is a row-wise read of T_i^T
#pragma unroll
    for (int cc = 0; cc < HC; ++cc) num[cc] = f32x16{};
    float den = 0.f;
#pragma unroll
    for (int k = 0; k < NS; ++k) {
      const bf16x8 pq = relu8(row_ok ? qv[k] : bf16x8{});
#pragma unroll
      for (int cc = 0; cc < HC; ++cc) {
        num[cc] = mfma32(rd_row(lb1, c0 + 32 * cc, k), pq, num[cc]);
      }
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) den += bf2f(pq[jj]) * zeta[16 * k + 8 * g + jj];
    }
    den = xor32_sum(den);
    inv_den = (topk < nb && den != 0.f) ? 1.f / den : 0.f;
  }
  if (!row_ok) return;
  const float a = alpha[(size_t)bh * N + row];
  const float ws = a * inv_l, wl = (1.f - a) * inv_den;
  float* orow = O + hoff + (size_t)row * D;
#pragma unroll
  for (int cc = 0; cc < HC; ++cc)
#pragma unroll
    for (int qd = 0; qd < 4; ++qd) {
      f32x4 v;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float x = oo[cc][4 * qd + e] * ws;
        v[e] = fmaf(num[cc][4 * qd + e], wl, x);
      }
      *reinterpret_cast<f32x4*>(orow + c0 + 32 * cc + 8 * qd + 4 * g) = v;
    }
}


template <class T, int D>
__global__ __launch_bounds__(kSplitThreads, 2) void split_kernel(
    const T* __restrict__ Q, const T* __restrict__ K, const T* __restrict__ V,
    const int32_t* __restrict__ idx, const float* __restrict__ alpha,
    const __bf16* __restrict__ t_g, const float* __restrict__ Z, const float* __restrict__ zb,
    float* __restrict__ O, int N, int nb, int topk, float c_log2) {
  using S_ = SplitShape<T, D>;
  __shared__ __attribute__((aligned(16))) __bf16 lq[S_::QBUF];
  __shared__ __attribute__((aligned(16))) __bf16 lb0[S_::BUF];
  __shared__ __attribute__((aligned(16))) __bf16 lb1[S_::BUF];
  const int w = threadIdx.x / kWave;
  const int item = xcd_remap(blockIdx.x, gridDim.x);
  const int bh = item / nb, qb = item % nb;
#define SLA_WAVE(QH_, KH_) \
  split_wave<T, D, QH_, KH_>(Q, K, V, idx, alpha, t_g, Z, zb, O, N, nb, topk, c_log2, lq, lb0, lb1, bh, qb)
  // one instantiation per wavefront quarter, so that its row, key and channel offsets are
  // compile-time constants (immediate LDS offsets instead of address registers)
  switch (w) {
    case 0: SLA_WAVE(0, 0); break;
    case 1: SLA_WAVE(1, 0); break;
    case 2: SLA_WAVE(0, 1); break;
    default: SLA_WAVE(1, 1); break;
  }
#undef SLA_WAVE
}

template <class T, int D>
hipError_t launch_split_t(const Dims& p, const void* Q, const void* K, const void* V,
                          const int32_t* idx, const float* alpha, const __bf16* t_bf,
                          const float* Z, const float* zb, float* O, hipStream_t stream) {
  const int total = p.B * p.H * p.nb;
  const float c_log2 = 1.4426950408889634f / sqrtf((float)D);
  split_kernel<T, D><<<total, kSplitThreads, 0, stream>>>(
      (const T*)Q, (const T*)K, (const T*)V, idx, alpha, t_bf, Z, zb, O, p.N, p.nb, p.topk,
      c_log2);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_sparse_tsel(const Dims& p, const void* Q, const void* K, const void* V,
                              const int32_t* idx, const float* alpha, const __bf16* t_bf,
                              const float* Z, const float* zb, float* O, hipStream_t stream) {
  if (p.dtype == kBF16 && p.d == 128)
    return launch_split_t<__bf16, 128>(p, Q, K, V, idx, alpha, t_bf, Z, zb, O, stream);
  if (p.dtype == kBF16 && p.d == 64)
    return launch_split_t<__bf16, 64>(p, Q, K, V, idx, alpha, t_bf, Z, zb, O, stream);
  if (p.dtype == kF32 && p.d == 128)
    return launch_split_t<float, 128>(p, Q, K, V, idx, alpha, t_bf, Z, zb, O, stream);
  return launch_split_t<float, 64>(p, Q, K, V, idx, alpha, t_bf, Z, zb, O, stream);
}

}  // namespace sla
