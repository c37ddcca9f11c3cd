// pisa.hip - the PISA exact-or-approximate attention forward on gfx950.
//
// Source: "PISA - Piecewise Sparse Attention per Efficient Diffusion Transformers", Italian
// technical summary, section 2: o_t = N_t / D_t where the kept key blocks S_i contribute exactly,
// every other block j by its zero-order term alpha_tj (sum of its values) with
// alpha_tj = exp(q_t kbar_j^T / sqrt(d)), and one global first-order correction
// (q_t / sqrt(d)) Hbar sum_{j not kept} alpha_tj is added to the numerator; the denominator gets
// r_j alpha_tj per unselected block (r_j its token count; the first-order term of the
// denominator vanishes at the centroid).  The fused kernel of that section interleaves an exact
// phase over the kept blocks, a scan of the blocks' aggregated vectors, and the correction
// inside one online softmax; this kernel does the same.
//
// One workgroup = query blocks 2p and 2p + 1 of one (batch, head), 256 threads, the same tile
// machinery as the two-block SLA2 kernel: wavefront w owns rows 32 (w % 2) .. + 31 of query
// block 2p + w / 2 (one query row per lane, Q in registers as the B operand of S^T = K Q^T).
//   exact phase   the ascending union of the two kept lists; each K_j, V_j tile is staged once
//                 into LDS for both blocks (double-buffered, direct-to-LDS loads for bf16 with
//                 d = 128) and each wavefront skips the tiles its block did not keep.  Online
//                 softmax in the log2 domain (the running maximum moves only by more than 2^8),
//                 P in bf16, row sums from the bf16 P, O^T += V^T P^T on bf16 MFMA.
//   scan phase    the key centroids kbar (bf16) and value sums vs (bf16) of all n_b blocks, 64 per
//                 tile, staged like K and V tiles and shared by both blocks.  The same S, P and
//                 PV steps with the centroids as keys and the value sums as values, in the same
//                 running softmax; a centroid is masked where the wavefront's block kept it or
//                 past n_b; its weight in the row sum is r_j (64, or the short last block's
//                 count); sum_U alpha is kept beside the row sum.
//   epilogue      Hbar^T (bf16) into LDS; num^T = Hbar^T Q^T by MFMA;
//                 O = (O_acc + num * sum_U alpha / sqrt(d)) / rowsum, fp32 stores, rows past N
//                 not stored.
// All kept blocks (topk == n_b) skip the scan: PISA is then exact attention.
#include <type_traits>

#include "sla_device.hpp"
#include "sla_launch.hpp"
#include "sla_tiles.hpp"

namespace sla {

namespace {

constexpr int kPisaThreads = 256;
constexpr int kPisaMaxWords = 64;  // bitmap words per query block: n_b <= 2048

template <class T>
__device__ __forceinline__ bf16x8 pisa_row8(const T* p);
template <>
__device__ __forceinline__ bf16x8 pisa_row8<__bf16>(const __bf16* p) {
  return *reinterpret_cast<const bf16x8*>(p);
}
template <>
__device__ __forceinline__ bf16x8 pisa_row8<float>(const float* p) {
  const f32x4 a = *reinterpret_cast<const f32x4*>(p);
  const f32x4 b = *reinterpret_cast<const f32x4*>(p + 4);
  return bf16x8{f2bf(a[0]), f2bf(a[1]), f2bf(a[2]), f2bf(a[3]),
                f2bf(b[0]), f2bf(b[1]), f2bf(b[2]), f2bf(b[3])};
}
// fp32 inputs: the bf16 remainder x - bf16(x) of 8 consecutive values (0 for bf16 inputs)
template <class T>
__device__ __forceinline__ bf16x8 pisa_row8_lo(const T* p) {
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
__device__ __forceinline__ float pisa_sum8(bf16x8 v, float acc) {
  const bf16x2 one = {f2bf(1.f), f2bf(1.f)};
#pragma unroll
  for (int i = 0; i < 4; ++i) acc = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{v[2 * i], v[2 * i + 1]}, one, acc, false);
  return acc;
}

constexpr float kPisaRescaleSlack = 8.f;  // log2 units
// the running maximum starts finite so that a fully masked tile gives P = 2^(-inf) = 0, never
// 2^(-inf + inf)
constexpr float kPisaMaxFloor = -1e30f;

template <class T, int D>
__global__ __launch_bounds__(kPisaThreads, 2) void pisa_kernel(
    const T* __restrict__ Q, const T* __restrict__ K, const T* __restrict__ V,
    const int32_t* __restrict__ idx, const __bf16* __restrict__ kbar_hi,
    const __bf16* __restrict__ kbar_lo, const __bf16* __restrict__ vsum,
    const __bf16* __restrict__ hbar_t, float* __restrict__ O, int N, int nb, int topk,
    float c_log2, float qscale) {
  constexpr int NS = D / 16;  // MFMA k-steps over the head dim
  constexpr int NC = D / 32;  // 32-channel output tiles
  constexpr int TILE = TileLayout<D>::ELEMS;
  constexpr bool SPLIT = sizeof(T) == 4;  // fp32 inputs: K (and kbar) as bf16 hi + lo tiles
  constexpr int TILES = SPLIT ? 3 : 2;    // per buffer: K (hi), V, [K lo]
  static_assert(D * TileLayout<D>::PITCH <= TILES * TILE, "Hbar^T must fit in one tile buffer");
  __shared__ __attribute__((aligned(16))) __bf16 lb0[TILES * TILE];
  __shared__ __attribute__((aligned(16))) __bf16 lb1[TILES * TILE];
  __shared__ uint32_t bm[2][kPisaMaxWords];  // kept-block bitmaps of the two query blocks
  __shared__ int32_t ul[kPisaMaxWords * 32];  // the union, ascending: (j << 2) | kept-by mask
  __shared__ int32_t ucount;
  auto buf = [&](auto BUFC) -> __bf16* { return decltype(BUFC)::value ? lb1 : lb0; };

  const int tid = threadIdx.x;
  const int lane = tid % kWave, g = lane / 32;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int item = xcd_remap(blockIdx.x, gridDim.x);
  const int npair = (nb + 1) / 2;
  const int bh = item / npair, pr = item % npair;
  const int qb0 = 2 * pr;
  const bool has1 = qb0 + 1 < nb;
  const int blk = wave / 2;
  const size_t hoff = (size_t)bh * N * D;
  const size_t soff = (size_t)bh * nb * D;  // this head's rows of kbar and vs
  const int nw = (nb + 31) / 32;

  // ---- kept-block bitmaps and their ascending union ----
  if (tid < 2 * kPisaMaxWords) bm[tid / kPisaMaxWords][tid % kPisaMaxWords] = 0u;
  __syncthreads();
  for (int t = tid; t < 2 * topk; t += kPisaThreads) {
    const int b = t / topk;
    if (b == 0 || has1) {
      const int j = idx[((size_t)bh * nb + qb0 + b) * topk + t % topk];
      atomicOr(&bm[b][j / 32], 1u << (j % 32));
    }
  }
  __syncthreads();
  if (wave == 0) {
    const uint32_t w0 = lane < nw ? bm[0][lane] : 0u, w1 = lane < nw ? bm[1][lane] : 0u;
    const uint32_t u = w0 | w1;
    const int cnt = __popc(u);
    int pos = cnt;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
      const int v = __shfl_up(pos, o);
      if (lane >= o) pos += v;
    }
    if (lane == kWave - 1) ucount = pos;
    pos -= cnt;
    for (uint32_t r = u; r; r &= r - 1) {
      const int b = __ffs(r) - 1;
      ul[pos++] = ((32 * lane + b) << 2) | (((w0 >> b) & 1u) ? 1 : 0) | (((w1 >> b) & 1u) ? 2 : 0);
    }
  }
  __syncthreads();
  const int nu = ucount;
  const int nct = topk < nb ? (nb + kBlock - 1) / kBlock : 0;  // centroid tiles of the scan
  const int total = nu + nct;
  const int nlast = N - (nb - 1) * kBlock;  // tokens of the last block

  // ---- staging: tiles t < nu are K_j, V_j of the union, tiles nu + ct centroids and value sums
  // of blocks 64 ct .. 64 ct + 63 ----
  constexpr bool DIRECT = sizeof(T) == 2 && D == 128;
  int f_next = 0, nv_next = kBlock;
  auto stage = [&](int t, auto BUFC) {
    __bf16* dst = buf(BUFC);
    if (t < nu) {
      const int e = ul[t];
      const int j = e >> 2;
      const int nv = min(kBlock, N - j * kBlock);
      const T* ksrc = K + hoff + (size_t)j * kBlock * D;
      const T* vsrc = V + hoff + (size_t)j * kBlock * D;
      f_next = e & 3;
      nv_next = nv;
      if constexpr (DIRECT) {
        if (nv == kBlock) {
          load_tile_direct<kPisaThreads>(ksrc, dst, tid);
          load_tile_direct<kPisaThreads>(vsrc, dst + TILE, tid);
        } else {
          load_tile_direct_clamped<kPisaThreads>(ksrc, dst, tid, nv);
          load_tile_direct_clamped<kPisaThreads>(vsrc, dst + TILE, tid, nv);
        }
      } else {
        TileLoader<T, D, kPisaThreads> lk, lv;
        lk.load(ksrc, nv, tid);
        lv.load(vsrc, nv, tid);
        if constexpr (SPLIT)
          lk.store_split(dst, dst + 2 * TILE, tid);
        else
          lk.store(dst, tid);
        lv.store(dst + TILE, tid);
      }
    } else {
      const int j0 = (t - nu) * kBlock;
      const int nv = min(kBlock, nb - j0);
      const __bf16* ksrc = kbar_hi + soff + (size_t)j0 * D;
      const __bf16* vsrc = vsum + soff + (size_t)j0 * D;
      f_next = 3;
      nv_next = nv;
      if constexpr (DIRECT) {
        if (nv == kBlock) {
          load_tile_direct<kPisaThreads>(ksrc, dst, tid);
          load_tile_direct<kPisaThreads>(vsrc, dst + TILE, tid);
        } else {
          load_tile_direct_clamped<kPisaThreads>(ksrc, dst, tid, nv);
          load_tile_direct_clamped<kPisaThreads>(vsrc, dst + TILE, tid, nv);
        }
      } else {
        TileLoader<__bf16, D, kPisaThreads> lk, lv;
        lk.load(ksrc, nv, tid);
        lv.load(vsrc, nv, tid);
        lk.store(dst, tid);
        lv.store(dst + TILE, tid);
        if constexpr (SPLIT) {
          TileLoader<__bf16, D, kPisaThreads> ll;
          ll.load(kbar_lo + soff + (size_t)j0 * D, nv, tid);
          ll.store(dst + 2 * TILE, tid);
        }
      }
    }
  };
  auto zero_tail = [&](auto BUFC, int nv) {
    if constexpr (DIRECT) {
      if (nv < kBlock) {
        zero_tile_rows<kPisaThreads>(buf(BUFC), tid, nv);
        zero_tile_rows<kPisaThreads>(buf(BUFC) + TILE, tid, nv);
        __syncthreads();
      }
    }
  };
  constexpr bool XADDR = D == 128;
  int ap_row = 0, ap_va = 0, ap_vb = 0;
  if constexpr (XADDR) {
    ap_row = row_part(lane);
    ap_va = tr_part<4>(lane, 0);
    ap_vb = tr_part<4>(lane, 8);
  }
  auto launder = [&]() {
    if constexpr (XADDR) asm volatile("" : "+v"(ap_row), "+v"(ap_va), "+v"(ap_vb));
  };
  auto rd_row = [&](const __bf16* tile, int R0, int k) -> bf16x8 {
    if constexpr (XADDR)
      return lds_row16(tile, R0 * 256 + (ap_row ^ (32 * k)));
    else
      return *reinterpret_cast<const bf16x8*>(tile + TileLayout<D>::off(R0 + lane % 32, 16 * k + 8 * g));
  };
  auto rd_tr_v = [&](const __bf16* tile, int row0, int col0) -> bf16x8 {
    if constexpr (XADDR)
      return join_tr(lds_tr_at(tile, row0 * 256 + (ap_va ^ (2 * col0))),
                     lds_tr_at(tile, row0 * 256 + (ap_vb ^ (2 * col0))));
    else
      return tr_operand<D, 4, 8>(tile, row0, col0, lane);
  };

  const int m = 32 * (wave % 2) + lane % 32;
  const int row = (qb0 + blk) * kBlock + m;
  const bool row_ok = row < N;
  bf16x8 q[NS], ql[SPLIT ? NS : 1];
  {
    const T* qr = Q + hoff + (size_t)min(row, N - 1) * D + 8 * g;
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      q[s] = row_ok ? pisa_row8<T>(qr + 16 * s) : bf16x8{};
      if constexpr (SPLIT) ql[s] = row_ok ? pisa_row8_lo<T>(qr + 16 * s) : bf16x8{};
    }
  }
  f32x16 os[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) os[c] = f32x16{};
  float mrun = kPisaMaxFloor, lsum = 0.f, asum = 0.f;

  // S^T of this wavefront's rows against the 64 keys of a staged tile
  auto scores = [&](const __bf16* Ks, f32x16* s) {
    bf16x8 ka[2][NS];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int k = 0; k < NS; ++k) ka[kt][k] = rd_row(Ks, 32 * kt, k);
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) s[kt] = f32x16{};
#pragma unroll
    for (int k = 0; k < NS; ++k)
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        if constexpr (SPLIT) {
          s[kt] = mfma32(rd_row(Ks + 2 * TILE, 32 * kt, k), q[k], s[kt]);
          s[kt] = mfma32(ka[kt][k], ql[k], s[kt]);
        }
        s[kt] = mfma32(ka[kt][k], q[k], s[kt]);
      }
  };
  // running maximum of the rows (log2 domain), rescaling O, the row sum and sum_U alpha
  auto update_max = [&](const f32x16* s) {
    float mx = -INFINITY;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[kt][i]);
    mx = xor32_max(mx) * c_log2;
    if (__ballot(mx > mrun + kPisaRescaleSlack)) {
      const float mnew = fmaxf(mrun, mx);
      const float corr = fast_exp2(mrun - mnew);
      mrun = mnew;
      lsum *= corr;
      asum *= corr;
#pragma unroll
      for (int c = 0; c < NC; ++c) os[c] *= corr;
    }
  };
  auto probs = [&](const f32x16* s, bf16x8* pb) -> float {
    float ps = 0.f;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) pb[u][jj] = f2bf(fast_exp2(fmaf(s[u / 2][8 * (u % 2) + jj], c_log2, -mrun)));
      ps = pisa_sum8(pb[u], ps);
    }
    return ps;
  };
  // V operands for PV (transposed reads), then O^T += V^T P^T; MFMA u covers keys 16u .. + 15
  auto read_v = [&](const __bf16* Vs, bf16x8 (&va)[NC][4]) {
#pragma unroll
    for (int c = 0; c < NC; ++c)
#pragma unroll
      for (int u = 0; u < 4; ++u) va[c][u] = rd_tr_v(Vs, 16 * u, 32 * c);
  };
  auto pv = [&](const bf16x8 (&va)[NC][4], const bf16x8* pb) {
#pragma unroll
    for (int c = 0; c < NC; ++c)
#pragma unroll
      for (int u = 0; u < 4; ++u) os[c] = mfma32(va[c][u], pb[u], os[c]);
  };

  using B0 = std::integral_constant<int, 0>;
  using B1 = std::integral_constant<int, 1>;
  int nv_cur = kBlock, f_cur = 0;
  if (total > 0) {
    stage(0, B0{});
    nv_cur = nv_next;
    f_cur = f_next;
    wait_vmem();
    __syncthreads();
    zero_tail(B0{}, nv_cur);
  }
  // every path into the loop has waited for the operands loaded into registers above (else the
  // compiler waits for all memory traffic, the next tile's prefetch included, in every step)
  wait_vmem();
  // the end of every step: tile t + 1 has landed in the other buffer
  auto finish = [&](int t, auto OTHERC) {
    nv_cur = nv_next;
    wait_vmem();
    __syncthreads();
    __builtin_amdgcn_sched_barrier(0);
    if (t + 1 < total) {
      f_cur = f_next;
      zero_tail(OTHERC, nv_cur);
    }
  };

  // exact phase: tile t of the union (MASK: the final union tile, the only one that can be short)
  auto step_exact = [&](int t, auto BUFC, auto MASKC) {
    constexpr int BUF = decltype(BUFC)::value;
    constexpr bool MASK = decltype(MASKC)::value;
    using OTHER = std::integral_constant<int, 1 - BUF>;
    const int nv = nv_cur;
    launder();
    if (t + 1 < total) stage(t + 1, OTHER{});
    if ((f_cur >> blk) & 1) {
      const __bf16* Ks = buf(BUFC);
      f32x16 s[2];
      scores(Ks, s);
      // V reads are independent of P: in unmasked steps they are issued before the softmax so
      // their LDS latency hides under it (the masked final step reads them after, staying
      // within registers)
      bf16x8 va[NC][4];
      if constexpr (!MASK) read_v(Ks + TILE, va);
      if (MASK && nv < kBlock) {
        const int lim = nv - 4 * g;
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
          for (int i = 0; i < 16; ++i)
            if (32 * kt + 8 * (i / 4) + i % 4 >= lim) s[kt][i] = -INFINITY;
      }
      update_max(s);
      bf16x8 pb[4];
      lsum += probs(s, pb);
      if constexpr (MASK) read_v(Ks + TILE, va);
      pv(va, pb);
    }
    finish(t, OTHER{});
  };

  // scan phase: centroid tile ct = t - nu
  auto step_scan = [&](int t, auto BUFC) {
    constexpr int BUF = decltype(BUFC)::value;
    using OTHER = std::integral_constant<int, 1 - BUF>;
    const int ct = t - nu;
    launder();
    if (t + 1 < total) stage(t + 1, OTHER{});
    {
      const __bf16* Ks = buf(BUFC);
      f32x16 s[2];
      scores(Ks, s);
      // mask the centroids this block keeps (computed exactly) and those past n_b; key of
      // register i in half kt: 32 kt + 8 (i / 4) + 4 g + i % 4
      const uint32_t m0 = bm[blk][2 * ct] >> (4 * g), m1 = bm[blk][2 * ct + 1] >> (4 * g);
      const int lim = nb - kBlock * ct - 4 * g;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int kk = 8 * (i / 4) + i % 4;
          const bool kept = (((kt ? m1 : m0) >> kk) & 1u) != 0u;
          if (kept || 32 * kt + kk >= lim) s[kt][i] = -INFINITY;
        }
      update_max(s);
      bf16x8 pb[4];
      const float ps = probs(s, pb);
      asum += ps;
      const int kl = nb - 1 - kBlock * ct;  // the last block's key slot in this tile
      if (nlast < kBlock && kl < kBlock) {
        // every centroid weighs r_j = 64 tokens except the short last block
        float pl = 0.f;
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
          for (int jj = 0; jj < 8; ++jj) {
            const int i = 8 * (u % 2) + jj;
            if (32 * (u / 2) + 8 * (i / 4) + 4 * g + i % 4 == kl) pl = bf2f(pb[u][jj]);
          }
        lsum += fmaf((float)kBlock, ps, -(float)(kBlock - nlast) * pl);
      } else {
        lsum = fmaf((float)kBlock, ps, lsum);
      }
      bf16x8 va[NC][4];
      read_v(Ks + TILE, va);
      pv(va, pb);
    }
    finish(t, OTHER{});
  };

  {
    using NoMask = std::integral_constant<bool, false>;
    using Mask = std::integral_constant<bool, true>;
    int t = 0;
    for (; t + 2 < nu; t += 2) {
      step_exact(t, B0{}, NoMask{});
      step_exact(t + 1, B1{}, NoMask{});
    }
    if (t + 1 < nu) {
      step_exact(t, B0{}, NoMask{});
      step_exact(t + 1, B1{}, Mask{});
    } else if (t < nu) {
      step_exact(t, B0{}, Mask{});
    }
    t = nu;
    if ((t & 1) && t < total) {
      step_scan(t, B1{});
      ++t;
    }
    for (; t + 1 < total; t += 2) {
      step_scan(t, B0{});
      step_scan(t + 1, B1{});
    }
    if (t < total) step_scan(t, B0{});
  }

  // ---- epilogue: Hbar^T [c][c'] into buffer 0 (free since the last step's barrier) ----
  {
    const __bf16* th = hbar_t + (size_t)bh * D * D;
#pragma unroll
    for (int half = 0; half < D / kBlock; ++half) {
      if constexpr (D == 128) {
        load_tile_direct<kPisaThreads>(th + half * kBlock * D, lb0 + half * kBlock * D, tid);
      } else {
        TileLoader<__bf16, D, kPisaThreads> ld;
        ld.load(th + half * kBlock * D, kBlock, tid);
        ld.store(lb0 + half * TILE, tid);
      }
    }
  }
  wait_vmem();
  __syncthreads();
  launder();
  const float ltot = xor32_sum(lsum);
  const float atot = xor32_sum(asum);
  const float inv_l = ltot > 0.f ? 1.f / ltot : 0.f;
  // num^T[c][m] = sum_c' Hbar^T[c][c'] q[m][c']
  f32x16 num[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) num[c] = f32x16{};
#pragma unroll
  for (int k = 0; k < NS; ++k)
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const bf16x8 a = rd_row(lb0, 32 * c, k);
      num[c] = mfma32(a, q[k], num[c]);
      if constexpr (SPLIT) num[c] = mfma32(a, ql[k], num[c]);
    }
  if (!row_ok) return;
  const float w1 = atot * qscale * inv_l;
  float* orow = O + hoff + (size_t)row * D;
#pragma unroll
  for (int c = 0; c < NC; ++c)
#pragma unroll
    for (int qd = 0; qd < 4; ++qd) {
      f32x4 v;
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = fmaf(num[c][4 * qd + e], w1, os[c][4 * qd + e] * inv_l);
      *reinterpret_cast<f32x4*>(orow + 32 * c + 8 * qd + 4 * g) = v;
    }
}

template <class T, int D>
hipError_t launch_pisa_t(const Dims& p, const void* Q, const void* K, const void* V,
                         const int32_t* idx, const __bf16* kbar_hi, const __bf16* kbar_lo,
                         const __bf16* vsum, const __bf16* hbar_t, float* O, hipStream_t stream) {
  const int total = p.B * p.H * ((p.nb + 1) / 2);
  const float qscale = 1.0f / sqrtf((float)D);
  const float c_log2 = 1.4426950408889634f * qscale;
  pisa_kernel<T, D><<<total, kPisaThreads, 0, stream>>>(
      (const T*)Q, (const T*)K, (const T*)V, idx, kbar_hi, kbar_lo, vsum, hbar_t, O, p.N, p.nb,
      p.topk, c_log2, qscale);
  return hipGetLastError();
}

}  // namespace

int pisa_max_blocks() { return kPisaMaxWords * 32; }

hipError_t launch_pisa(const Dims& p, const void* Q, const void* K, const void* V,
                       const int32_t* idx, const __bf16* kbar_hi, const __bf16* kbar_lo,
                       const __bf16* vsum, const __bf16* hbar_t, float* O, hipStream_t stream) {
  if (p.nb > kPisaMaxWords * 32) return hipErrorInvalidValue;
  if (p.dtype == kBF16 && p.d == 128)
    return launch_pisa_t<__bf16, 128>(p, Q, K, V, idx, kbar_hi, kbar_lo, vsum, hbar_t, O, stream);
  if (p.dtype == kBF16 && p.d == 64)
    return launch_pisa_t<__bf16, 64>(p, Q, K, V, idx, kbar_hi, kbar_lo, vsum, hbar_t, O, stream);
  if (p.dtype == kF32 && p.d == 128)
    return launch_pisa_t<float, 128>(p, Q, K, V, idx, kbar_hi, kbar_lo, vsum, hbar_t, O, stream);
  return launch_pisa_t<float, 64>(p, Q, K, V, idx, kbar_hi, kbar_lo, vsum, hbar_t, O, stream);
}

}  // namespace sla
