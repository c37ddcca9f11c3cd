// sparse_pair.hip - block-sparse softmax branch and alpha combine on gfx950 for two query blocks
// per workgroup, with the linear branch's per-query-block state T_i = sum_{j not in sel(i)} h_j
// taken from memory (formed for every query block at once by the mask-product kernel,
// linear_gemm.hip).
//
// Sources: SLA2 Italian summary sections 1 and 2.A and Arabic summary sections 1 and 2.alef
// (sparse branch renormalised over the kept blocks; O = alpha O_s + (1 - alpha) O_l); SALAD
// section 2 (ReLU feature map of the linear branch, over the blocks the sparse branch leaves).
//
// One workgroup = two query blocks of one (batch, head): 2p and 2p + 1, or (the mask-product
// forward) the pair that pair_match_kernel below chose among nearby blocks for the most kept
// key blocks in common.  Nearby query blocks keep mostly the same key blocks, so the workgroup
// walks the ascending union of their two index lists and stages each K_j, V_j tile into LDS
// once for both: every tile byte read from L2 serves up to 128 query rows instead of 64.
// Wavefront w takes rows 32 (w % 2) .. + 31 of the pair's block w / 2 against all 64 keys of a
// tile, and skips the tiles its block did not keep
// (the result is exactly each block's own sparse branch).  Per tile: S^T = K_j Q^T
// (v_mfma_f32_32x32x16_bf16, Q in registers as the B operand, so each lane owns one query row
// and the row statistics stay in-lane), online softmax in the log2 domain (the running maximum
// only moves when a row's maximum grows by more than 2^8), P rounded to bf16, row sums from the
// bf16 P with v_dot2, O_s^T += V_j^T P^T with V read transposed from LDS (ds_read_b64_tr_b16).
// K_j, V_j tiles are double-buffered in LDS, one array per buffer so that the compiler can tell
// the buffer being filled by direct-to-LDS loads from the one being read.  bf16 tiles with
// d = 128 come through per-head buffer resources (buffer_load_dwordx4 ... lds): the tile offset
// is a scalar register and each lane's offset a fixed VGPR, so staging a tile costs no per-lane
// address arithmetic (a head spans at most 2048 x 64 x 128 x 2 bytes, inside the 32-bit range);
// the short last tile of a sequence takes its offsets in the range-checked vector part, so it
// reads zeros past N, never past the tensor.
// Epilogue: T_i^T (bf16, [c][c']) of each block is loaded into a tile buffer, zeta_i = Z -
// sum_kept z_j; each wavefront computes num = relu(Q) T_i by MFMA, den = relu(q) . zeta_i, and
// O = alpha O_s / l + (1 - alpha) num / den (the linear part is 0 when nothing is unselected or
// den == 0), fp32 stores; rows past N are not stored.
#include <type_traits>

#include "sla_device.hpp"
#include "sla_launch.hpp"
#include "sla_tiles.hpp"

namespace sla {

namespace {

constexpr int kPairThreads = 256;
constexpr int kPairMaxWords = 64;  // bitmap words of the union: n_b <= 2048
// XCDs per head of the pair kernel's grid (xcd_group_map): 4 by default, each head's pairs
// shared by the XCDs of one half of the chip, the heads alternating between the halves (an XCD
// works through a larger share of fewer heads, which its L2 holds better); 8 (every XCD takes an
// eighth of every head) when branch dropping may leave heads with unequal work, so that no half
// of the chip idles while the other finishes its heads
__host__ __device__ __forceinline__ bool pair_map(int xg, int wg, int heads, int npair, int* bh, int* pr) {
  return xg == 8 ? xcd_group_map<8>(wg, heads, npair, bh, pr) : xcd_group_map<4>(wg, heads, npair, bh, pr);
}
__host__ __device__ __forceinline__ int pair_id(int xg, int bh, int pr, int npair) {
  return xg == 8 ? xcd_group_id<8>(bh, pr, npair) : xcd_group_id<4>(bh, pr, npair);
}
__host__ __device__ __forceinline__ int pair_grid(int xg, int heads, int npair) {
  return xg == 8 ? xcd_group_grid<8>(heads, npair) : xcd_group_grid<4>(heads, npair);
}
inline int pair_xg(bool unequal_heads) { return unequal_heads ? 8 : 4; }

template <class T>
__device__ __forceinline__ bf16x8 pair_row8(const T* p);
template <>
__device__ __forceinline__ bf16x8 pair_row8<__bf16>(const __bf16* p) {
  return *reinterpret_cast<const bf16x8*>(p);
}
template <>
__device__ __forceinline__ bf16x8 pair_row8<float>(const float* p) {
  const f32x4 a = *reinterpret_cast<const f32x4*>(p);
  const f32x4 b = *reinterpret_cast<const f32x4*>(p + 4);
  return bf16x8{f2bf(a[0]), f2bf(a[1]), f2bf(a[2]), f2bf(a[3]),
                f2bf(b[0]), f2bf(b[1]), f2bf(b[2]), f2bf(b[3])};
}

// fp32 inputs: the bf16 remainder x - bf16(x) of 8 consecutive values (0 for bf16 inputs)
template <class T>
__device__ __forceinline__ bf16x8 pair_row8_lo(const T* p) {
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
__device__ __forceinline__ float pair_sum8(bf16x8 v, float acc) {
  const bf16x2 one = {f2bf(1.f), f2bf(1.f)};
#pragma unroll
  for (int i = 0; i < 4; ++i) acc = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{v[2 * i], v[2 * i + 1]}, one, acc, false);
  return acc;
}

constexpr float kPairRescaleSlack = 8.f;  // log2 units: P may reach 2^8 before the maximum moves

// TRAIN: also write what the backward needs per query row (TrainRows, sla_launch.hpp): the
// normalised branches O_s and O_l, the sparse branch's log2-sum-exp2 and 1 / den (0 where the
// linear branch is defined as 0)
// SOFT (the SoftTop-k training path): every key block is walked, the tile of key block j
// weighted by msoft[query block][j] in the sparse branch (P = M_ij 2^(S c - m)), and the
// linear branch's zeta_i = Z - sum_j M_ij z_j (T_i from the weighted mask GEMM); idx is unused.
template <class T, int D, bool TRAIN, bool SOFT = false>
__global__ __launch_bounds__(kPairThreads, 2) void pair_kernel(
    const T* __restrict__ Q, const T* __restrict__ K, const T* __restrict__ V,
    const int32_t* __restrict__ idx, const float* __restrict__ alpha,
    const __bf16* __restrict__ t_g, const float* __restrict__ Z, const float* __restrict__ zb,
    float* __restrict__ O, int N, int nb, int topk, float c_log2, int heads, int xg,
    const uint32_t* __restrict__ flags, TrainRows tr, const int32_t* __restrict__ out_rows,
    const float* __restrict__ msoft = nullptr, const int32_t* __restrict__ order = nullptr,
    const int32_t* __restrict__ pairs = nullptr) {
  constexpr int NS = D / 16;  // MFMA k-steps over the head dim
  constexpr int NC = D / 32;  // 32-channel output tiles
  constexpr int TILE = TileLayout<D>::ELEMS;
  // fp32 inputs keep K as bf16 hi + lo tiles so that S = K Q^T is about fp32-accurate
  // (Kh Qh + Kh Ql + Kl Qh); bf16 inputs are exact in one bf16 tile
  constexpr bool SPLIT = sizeof(T) == 4;
  constexpr int TILES = SPLIT ? 3 : 2;  // per buffer: K (hi), V, [K lo]
  static_assert(D * TileLayout<D>::PITCH <= TILES * TILE, "T^T must fit in one tile buffer");
  __shared__ __attribute__((aligned(16))) __bf16 lb0[TILES * TILE];
  __shared__ __attribute__((aligned(16))) __bf16 lb1[TILES * TILE];
  __shared__ uint32_t bm[2][kPairMaxWords];  // kept-block bitmaps of the two query blocks
  __shared__ int32_t ul[kPairMaxWords * 32];  // the union, ascending: (j << 2) | kept-by mask
  __shared__ int32_t ucount;
  __shared__ float zeta[2][D];
  auto buf = [&](auto BUFC) -> __bf16* { return decltype(BUFC)::value ? lb1 : lb0; };

  const int tid = threadIdx.x;
  const int lane = tid % kWave, g = lane / 32;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);  // wavefront-uniform (scalar branches)
  // each head's pairs are split evenly among the XCDs of its group (heads may differ in work
  // when a branch is dropped); the grid's padding workgroups exit here, before any barrier
  const int npair = (nb + 1) / 2;
  int bh, pr;
  // order (optional): the workgroup ids in dispatch order, each XCD's own items largest union
  // first (pair_order_kernel), so that the shortest workgroups fill the end of the launch
  const int wg = order ? order[blockIdx.x] : (int)blockIdx.x;
  if (!pair_map(xg, wg, heads, npair, &bh, &pr)) return;
  // the two query blocks: 2p and 2p + 1, or (pairs) the ones matched by overlap of their kept
  // sets; an odd n_b (or an odd matching window) leaves one workgroup one block, whose absent
  // second block is given the id n_b (all its rows lie past N)
  int qa = 2 * pr, qbv = 2 * pr + 1;
  if (pairs) {
    qa = pairs[2 * ((size_t)bh * npair + pr)];
    qbv = pairs[2 * ((size_t)bh * npair + pr) + 1];
  }
  const bool has1 = pairs ? qbv >= 0 : qbv < nb;
  const int qb1 = has1 ? qbv : nb;
  auto qsel = [&](int b) { return b ? qb1 : qa; };
  const int blk = wave / 2;  // this wavefront's query block: qsel(blk)
  const size_t hoff = (size_t)bh * N * D;
  const int nw = (nb + 31) / 32;

  // ---- the union of the two ascending index lists, with the kept-by bits ----
  if constexpr (SOFT) {  // every key block, weighted for both query blocks
    for (int t = tid; t < nb; t += kPairThreads) ul[t] = (t << 2) | 3;
    if (tid == 0) ucount = nb;
  }
  if (tid < 2 * kPairMaxWords) bm[tid / kPairMaxWords][tid % kPairMaxWords] = 0u;
  __syncthreads();
  for (int t = tid; !SOFT && t < 2 * topk; t += kPairThreads) {
    const int b = t / topk;
    if (b == 0 || has1) {
      const int j = idx[((size_t)bh * nb + qsel(b)) * topk + t % topk];
      atomicOr(&bm[b][j / 32], 1u << (j % 32));
    }
  }
  __syncthreads();
  if (!SOFT && wave == 0) {
    const uint32_t w0 = lane < nw ? bm[0][lane] : 0u, w1 = lane < nw ? bm[1][lane] : 0u;
    const uint32_t u = w0 | w1;
    const int cnt = __popc(u);
    int pos = cnt;  // inclusive prefix sum over the lanes
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
  // branch dropping (workgroup-uniform): a dropped sparse branch walks no tiles, a dropped
  // linear branch loads no state
  const uint32_t fl = flags ? flags[bh] : 0u;
  const bool lin = !(fl & kDropLinear);
  const int nu = (fl & kDropSparse) ? 0 : ucount;

  // Tile staging: every thread moves its share of each tile.  bf16 tiles with d = 128 and all
  // 64 rows valid go HBM -> LDS directly (no registers), issued at the start of the iteration
  // that uses the other buffer; other tiles (fp32 inputs, d = 64, the short last block) go
  // through registers with zero fill, stored right away.  z_j travels with the tile: threads
  // tid < D keep the sum over the first block's kept tiles, threads D .. 2D - 1 the second's.
  constexpr bool DIRECT = sizeof(T) == 2 && D == 128;
  // DIRECT tiles come through per-head buffer resources: the tile offset is a scalar, each
  // lane's offset inside a tile a fixed register, and the short last tile's rows past N read as
  // zero
  const __amdgpu_buffer_rsrc_t rk = make_rsrc(K + hoff, (uint32_t)((size_t)N * D * sizeof(T)));
  const __amdgpu_buffer_rsrc_t rv = make_rsrc(V + hoff, (uint32_t)((size_t)N * D * sizeof(T)));
  const uint32_t lane_voff = DIRECT ? tile_lane_voff<kPairThreads>(tid) : 0u;
  const int zb_blk = tid / D;  // 0, 1 for tid < 2D
  const bool z_lane = tid < 2 * D;
  float z_in = 0.f;       // z_j of the tile being staged
  int f_next = 0;         // kept-by bits of the tile being staged
  int nv_next = kBlock;   // valid rows of the tile being staged
  float zacc = 0.f;
  auto stage = [&](int t, auto BUFC) {
    const int e = ul[t];
    const int j = e >> 2;
    const int nv = min(kBlock, N - j * kBlock);
    __bf16* dst = buf(BUFC);
    const T* ksrc = K + hoff + (size_t)j * kBlock * D;
    const T* vsrc = V + hoff + (size_t)j * kBlock * D;
    if (z_lane) z_in = zb[((size_t)bh * nb + j) * D + tid % D];
    if constexpr (SOFT) {
      if (z_lane) z_in *= msoft[((size_t)bh * nb + min(qsel(zb_blk), nb - 1)) * nb + j];
    }
    f_next = e & 3;
    nv_next = nv;
    if constexpr (DIRECT) {
      // a short tile (the last block of the sequence) reads zeros past N, and its tail rows are
      // zeroed again after the loads land (zero_tail), so no register path sits in the loop
      const uint32_t toff = (uint32_t)__builtin_amdgcn_readfirstlane(j) * (uint32_t)(kBlock * D * sizeof(T));
      load_tile_buf<kPairThreads>(rk, lane_voff, toff, dst, tid, nv < kBlock);
      load_tile_buf<kPairThreads>(rv, lane_voff, toff, dst + TILE, tid, nv < kBlock);
    } else {
      TileLoader<T, D, kPairThreads> lk, lv;
      lk.load(ksrc, nv, tid);
      lv.load(vsrc, nv, tid);
      if constexpr (SPLIT)
        lk.store_split(dst, dst + 2 * TILE, tid);
      else
        lk.store(dst, tid);
      lv.store(dst + TILE, tid);
    }
  };
  // DIRECT tiles with fewer than 64 valid rows: zero the tail once every load has landed and
  // been published by a barrier (workgroup-uniform condition; at most once per head)
  auto zero_tail = [&](auto BUFC, int nv) {
    if constexpr (DIRECT) {
      if (nv < kBlock) {
        zero_tile_rows<kPairThreads>(buf(BUFC), tid, nv);
        zero_tile_rows<kPairThreads>(buf(BUFC) + TILE, tid, nv);
        __syncthreads();
      }
    }
  };
  // LDS operand reads.  d = 128: per-lane address parts computed once and laundered through an
  // empty asm at the start of every tile (so the compiler re-derives the per-block addresses
  // with one v_xor each instead of holding dozens of them in registers across the loop); row
  // and buffer offsets are immediates.  d = 64: the padded layout's plain offsets.
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
  // row-wise operand: row R0 + lane%32 (R0 % 32 == 0), channels 16k + 8g .. + 7
  auto rd_row = [&](const __bf16* tile, int R0, int k) -> bf16x8 {
    if constexpr (XADDR)
      return lds_row16(tile, R0 * 256 + (ap_row ^ (32 * k)));
    else
      return *reinterpret_cast<const bf16x8*>(tile + TileLayout<D>::off(R0 + lane % 32, 16 * k + 8 * g));
  };
  // transposed operand in PV key order (step 4, gap 8)
  auto rd_tr_v = [&](const __bf16* tile, int row0, int col0) -> bf16x8 {
    if constexpr (XADDR)
      return join_tr(lds_tr_at(tile, row0 * 256 + (ap_va ^ (2 * col0))),
                     lds_tr_at(tile, row0 * 256 + (ap_vb ^ (2 * col0))));
    else
      return tr_operand<D, 4, 8>(tile, row0, col0, lane);
  };

  // Q of this wavefront's 32 rows as the B operand of S^T = K Q^T: k-slot 8g + jj of step s <->
  // channel 16s + 8g + jj (rows past N, and the absent second block of an odd n_b, read a
  // clamped row and are zeroed)
  const int m = 32 * (wave % 2) + lane % 32;
  const int row = qsel(blk) * kBlock + m;
  const bool row_ok = row < N;
  bf16x8 q[NS], ql[SPLIT ? NS : 1];
  {
    const T* qr = Q + hoff + (size_t)min(row, N - 1) * D + 8 * g;
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      q[s] = row_ok ? pair_row8<T>(qr + 16 * s) : bf16x8{};
      if constexpr (SPLIT) ql[s] = row_ok ? pair_row8_lo<T>(qr + 16 * s) : bf16x8{};
    }
  }
  f32x16 os[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) os[c] = f32x16{};
  float mrun = -INFINITY, lsum = 0.f;

  using B0 = std::integral_constant<int, 0>;
  using B1 = std::integral_constant<int, 1>;
  int nv_cur = kBlock, f_cur = 0;
  if (nu > 0) {
    stage(0, B0{});
    if (z_lane && ((f_next >> zb_blk) & 1)) zacc += z_in;
    nv_cur = nv_next;
    f_cur = f_next;
    wait_vmem();
    __syncthreads();
    zero_tail(B0{}, nv_cur);
  }
  // every path into the loop has waited for the Q operands (loaded above into registers):
  // otherwise the compiler cannot tell and waits for all memory traffic, the prefetch of the
  // next tile included, before the first MFMA of every step
  wait_vmem();
  // one tile of the union; BUF (= t & 1, a compile-time constant through the unrolled pair
  // below) is the buffer holding tile t, and tile t + 1 is staged into the other one (last read
  // in iteration t - 1).  MASK: the tile may be short (only the last block of the sequence is,
  // and it comes last in the ascending union), so only the final step carries the key mask
  // (the compiler turns it into selects on every key otherwise)
  auto step = [&](int t, auto BUFC, auto MASKC) {
    constexpr int BUF = decltype(BUFC)::value;
    constexpr bool MASK = decltype(MASKC)::value;
    const int nv = nv_cur;
    launder();
    if (t + 1 < nu) stage(t + 1, std::integral_constant<int, 1 - BUF>{});
    if ((f_cur >> blk) & 1) {  // this wavefront's block kept the tile (wavefront-uniform)
      // SOFT: this wavefront's block's weight of key block t (the union is every block in order)
      const float wgt = SOFT ? msoft[((size_t)bh * nb + min(qsel(blk), nb - 1)) * nb + t] : 1.f;
      const __bf16* Ks = buf(BUFC);
      const __bf16* Vs = Ks + TILE;
      // K operands of both 32-key halves, issued together ahead of their MFMAs
      bf16x8 ka[2][NS];
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int k = 0; k < NS; ++k) ka[kt][k] = rd_row(Ks, 32 * kt, k);
      f32x16 s[2];
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
      // V operands for PV: independent of P, so their LDS latency hides under the softmax (in
      // the masked final step they are read after it, which keeps that step within registers)
      bf16x8 va[NC][4];
      auto read_v = [&]() {
#pragma unroll
        for (int c = 0; c < NC; ++c)
#pragma unroll
          for (int u = 0; u < 4; ++u) va[c][u] = rd_tr_v(Vs, 16 * u, 32 * c);
      };
      if constexpr (!MASK) read_v();
      // key of accumulator register i in half kt: 32kt + 8(i/4) + 4g + i%4
      if (MASK && nv < kBlock) {
        const int lim = nv - 4 * g;
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
          for (int i = 0; i < 16; ++i)
            if (32 * kt + 8 * (i / 4) + i % 4 >= lim) s[kt][i] = -INFINITY;
      }
      float mx = -INFINITY;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[kt][i]);
      mx = xor32_max(mx) * c_log2;
      if (__ballot(mx > mrun + kPairRescaleSlack)) {
        const float mnew = fmaxf(mrun, mx);
        const float corr = fast_exp2(mrun - mnew);
        mrun = mnew;
        lsum *= corr;
#pragma unroll
        for (int c = 0; c < NC; ++c) os[c] *= corr;
      }
      bf16x8 pb[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) {
          const float pe = fast_exp2(fmaf(s[u / 2][8 * (u % 2) + jj], c_log2, -mrun));
          pb[u][jj] = f2bf(SOFT ? wgt * pe : pe);
        }
        lsum = pair_sum8(pb[u], lsum);
      }
      if constexpr (MASK) read_v();
      // O^T += V^T P^T ; MFMA u covers keys 16u .. 16u + 15
#pragma unroll
      for (int c = 0; c < NC; ++c)
#pragma unroll
        for (int u = 0; u < 4; ++u) os[c] = mfma32(va[c][u], pb[u], os[c]);
    }
    nv_cur = nv_next;
    wait_vmem();
    __syncthreads();
    // z_j and the kept-by bits of tile t + 1 are used only now, after the explicit wait above:
    // used earlier, the compiler would wait for every in-flight tile load at that point
    __builtin_amdgcn_sched_barrier(0);
    if (t + 1 < nu) {
      if (z_lane && ((f_next >> zb_blk) & 1)) zacc += z_in;
      f_cur = f_next;
      zero_tail(std::integral_constant<int, 1 - BUF>{}, nv_cur);
    }
  };
  {
    using NoMask = std::integral_constant<bool, false>;
    using Mask = std::integral_constant<bool, true>;
    int t = 0;
    for (; t + 2 < nu; t += 2) {
      step(t, B0{}, NoMask{});
      step(t + 1, B1{}, NoMask{});
    }
    if (t + 1 < nu) {
      step(t, B0{}, NoMask{});
      step(t + 1, B1{}, Mask{});
    } else if (t < nu) {
      step(t, B0{}, Mask{});
    }
  }

  // a dropped sparse branch staged no tiles, so the kept blocks' z_j are summed here
  if ((fl & kDropSparse) && lin && z_lane && (zb_blk == 0 || has1)) {
    const int32_t* il = idx + ((size_t)bh * nb + qsel(zb_blk)) * topk;
    for (int t = 0; t < topk; ++t) zacc += zb[((size_t)bh * nb + il[t]) * D + tid % D];
  }
  // ---- epilogue: T_i^T [c][c'] of block b into tile buffer b (both free since the last
  // step's barrier), in the tile row layout; zeta of each block ----
  if (lin) {
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      const __bf16* th = t_g + ((size_t)bh * nb + min(qsel(b), nb - 1)) * D * D;
      __bf16* dst = b ? lb1 : lb0;
#pragma unroll
      for (int half = 0; half < D / kBlock; ++half) {
        if constexpr (D == 128) {
          load_tile_direct<kPairThreads>(th + half * kBlock * D, dst + half * kBlock * D, tid);
        } else {
          TileLoader<__bf16, D, kPairThreads> ld;
          ld.load(th + half * kBlock * D, kBlock, tid);
          ld.store(dst + half * TILE, tid);
        }
      }
    }
    if (z_lane) zeta[zb_blk][tid % D] = Z[(size_t)bh * D + tid % D] - zacc;
    wait_vmem();
    __syncthreads();
    launder();
  }
  const float ltot = xor32_sum(lsum);
  const float inv_l = ltot > 0.f ? 1.f / ltot : 0.f;
  // num^T[c][m] = sum_c' T_i^T[c][c'] relu(Q)[m][c']: the A operand (rows c, k = c') is a
  // row-wise read of T_i^T
  const __bf16* tt = blk ? lb1 : lb0;
  f32x16 num[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) num[c] = f32x16{};
  float den = 0.f;
  if (lin) {
#pragma unroll
    for (int k = 0; k < NS; ++k) {
      const bf16x8 pq = relu8(q[k]);
#pragma unroll
      for (int c = 0; c < NC; ++c) num[c] = mfma32(rd_row(tt, 32 * c, k), pq, num[c]);
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) den += bf2f(pq[jj]) * zeta[blk][16 * k + 8 * g + jj];
    }
    den = xor32_sum(den);
  }
  const float inv_den = (lin && (SOFT || topk < nb) && den != 0.f) ? 1.f / den : 0.f;
  if (!row_ok) return;
  const float a = alpha[(size_t)bh * N + row];
  const float ws = a * inv_l, wl = (1.f - a) * inv_den;
  // out_rows entries are clamped to the sequence: a malformed permutation misplaces rows but
  // never writes outside O
  const int orow_i = out_rows ? min(max(out_rows[(size_t)bh * N + row], 0), N - 1) : row;
  float* orow = O + hoff + (size_t)orow_i * D;
#pragma unroll
  for (int c = 0; c < NC; ++c)
#pragma unroll
    for (int qd = 0; qd < 4; ++qd) {
      f32x4 v;
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = fmaf(num[c][4 * qd + e], wl, os[c][4 * qd + e] * ws);
      *reinterpret_cast<f32x4*>(orow + 32 * c + 8 * qd + 4 * g) = v;
    }
  if constexpr (TRAIN) {
    float* srow = tr.Os + hoff + (size_t)row * D;
    float* lrow = tr.Ol + hoff + (size_t)row * D;
#pragma unroll
    for (int c = 0; c < NC; ++c)
#pragma unroll
      for (int qd = 0; qd < 4; ++qd) {
        f32x4 vs, vl;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          vs[e] = os[c][4 * qd + e] * inv_l;
          vl[e] = num[c][4 * qd + e] * inv_den;
        }
        *reinterpret_cast<f32x4*>(srow + 32 * c + 8 * qd + 4 * g) = vs;
        *reinterpret_cast<f32x4*>(lrow + 32 * c + 8 * qd + 4 * g) = vl;
      }
    if (g == 0) {
      // a row with no kept key has no sparse probabilities: +inf makes every recomputed P 0
      tr.lse2[(size_t)bh * N + row] = ltot > 0.f ? mrun + __log2f(ltot) : INFINITY;
      tr.rden[(size_t)bh * N + row] = inv_den;
    }
  }
}

template <class T, int D>
hipError_t launch_pair_t(const Dims& p, const void* Q, const void* K, const void* V,
                         const int32_t* idx, const float* alpha, const __bf16* t_bf,
                         const float* Z, const float* zb, float* O, hipStream_t stream,
                         const uint32_t* flags, const TrainRows* tr, const int32_t* out_rows,
                         const int32_t* order, const int32_t* pairs) {
  const int xg = pair_xg(flags != nullptr);
  const int total = pair_grid(xg, p.B * p.H, (p.nb + 1) / 2);
  const float c_log2 = 1.4426950408889634f / sqrtf((float)D);
  if (tr)
    pair_kernel<T, D, true><<<total, kPairThreads, 0, stream>>>(
        (const T*)Q, (const T*)K, (const T*)V, idx, alpha, t_bf, Z, zb, O, p.N, p.nb, p.topk,
        c_log2, p.B * p.H, xg, flags, *tr, out_rows, nullptr, order, pairs);
  else
    pair_kernel<T, D, false><<<total, kPairThreads, 0, stream>>>(
        (const T*)Q, (const T*)K, (const T*)V, idx, alpha, t_bf, Z, zb, O, p.N, p.nb, p.topk,
        c_log2, p.B * p.H, xg, flags, TrainRows{}, out_rows, nullptr, order, pairs);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_sparse_soft(const Dims& p, const void* Q, const void* K, const void* V,
                              const float* msoft, const float* alpha, const __bf16* t_bf,
                              const float* Z, const float* zb, float* O, hipStream_t stream,
                              const TrainRows* tr) {
  if (p.nb > kPairMaxWords * 32 || p.dtype != kBF16 || p.d != 128 || !msoft) return hipErrorInvalidValue;
  const int total = pair_grid(4, p.B * p.H, (p.nb + 1) / 2);
  const float c_log2 = 1.4426950408889634f / sqrtf(128.f);
  if (tr)
    pair_kernel<__bf16, 128, true, true><<<total, kPairThreads, 0, stream>>>(
        (const __bf16*)Q, (const __bf16*)K, (const __bf16*)V, nullptr, alpha, t_bf, Z, zb, O, p.N, p.nb,
        p.nb, c_log2, p.B * p.H, 4, nullptr, *tr, nullptr, msoft);
  else
    pair_kernel<__bf16, 128, false, true><<<total, kPairThreads, 0, stream>>>(
        (const __bf16*)Q, (const __bf16*)K, (const __bf16*)V, nullptr, alpha, t_bf, Z, zb, O, p.N, p.nb,
        p.nb, c_log2, p.B * p.H, 4, nullptr, TrainRows{}, nullptr, msoft);
  return hipGetLastError();
}

hipError_t launch_sparse_pair(const Dims& p, const void* Q, const void* K, const void* V,
                              const int32_t* idx, const float* alpha, const __bf16* t_bf,
                              const float* Z, const float* zb, float* O, hipStream_t stream,
                              const uint32_t* flags, const TrainRows* tr,
                              const int32_t* out_rows, const int32_t* order,
                              const int32_t* pairs) {
  if (p.nb > kPairMaxWords * 32) return hipErrorInvalidValue;
  if (p.dtype == kBF16 && p.d == 128)
    return launch_pair_t<__bf16, 128>(p, Q, K, V, idx, alpha, t_bf, Z, zb, O, stream, flags, tr, out_rows, order, pairs);
  if (tr) return hipErrorInvalidValue;  // the training outputs exist for bf16, d = 128 only
  if (p.dtype == kBF16 && p.d == 64)
    return launch_pair_t<__bf16, 64>(p, Q, K, V, idx, alpha, t_bf, Z, zb, O, stream, flags, nullptr, out_rows, order, pairs);
  if (p.dtype == kF32 && p.d == 128)
    return launch_pair_t<float, 128>(p, Q, K, V, idx, alpha, t_bf, Z, zb, O, stream, flags, nullptr, out_rows, order, pairs);
  return launch_pair_t<float, 64>(p, Q, K, V, idx, alpha, t_bf, Z, zb, O, stream, flags, nullptr, out_rows, order, pairs);
}

// The pair kernel's dispatch order: each XCD's items (the workgroup ids wg with wg % 8 == x),
// within each head by the size of their union of kept blocks (from pair_match_kernel), largest
// first; ids that run nothing (past a short chunk, or a padding head) go last.
//   pair_order_kernel  one workgroup per (XCD, head of its group): that XCD's ids of the head,
//                      their sizes staged in LDS and ranked, largest first (a stable rank);
//                      the order changes which workgroup runs when, never what one computes.
constexpr int kOrderMax = 256;  // ids per (XCD, head): ceil(ceil(n_b / 2) / xg) <= 256

__global__ __launch_bounds__(kOrderMax) void pair_order_kernel(const int32_t* __restrict__ size, int heads,
                                                              int npair, int smax, int xg,
                                                              int32_t* __restrict__ order) {
  __shared__ int sz[kOrderMax];
  const int x = blockIdx.x, g0 = blockIdx.y * smax, t = threadIdx.x;
  const int id = 8 * (g0 + t) + x;
  if (t < smax) {
    int bh, pr;
    sz[t] = pair_map(xg, id, heads, npair, &bh, &pr) ? size[id] : -1;
  }
  __syncthreads();
  if (t >= smax) return;
  const int my = sz[t];
  int rank = 0;
  for (int j = 0; j < smax; ++j) {
    const int o = sz[j];
    rank += (o > my || (o == my && j < t)) ? 1 : 0;
  }
  order[8 * (g0 + rank) + x] = id;
}

int pair_order_ints(const Dims& p) {
  const int a = pair_grid(4, p.B * p.H, (p.nb + 1) / 2), b = pair_grid(8, p.B * p.H, (p.nb + 1) / 2);
  return a > b ? a : b;
}

// Query blocks paired by the overlap of their kept sets.  Windows of kMatchWin consecutive query
// blocks (neighbouring blocks are the ones that share kept blocks, and a window's pairs stay
// next to each other in the launch, sharing L2); inside a window, greedily, the two unpaired
// blocks with the most kept blocks in common (ties: the lowest pair of indices), until at most
// one is left (an odd last window: that block goes alone, second id -1).  Window w fills pair
// slots 16 w ..; the union a pair walks is |K_a| + |K_b| - |K_a & K_b|, so the most shared
// blocks make the shortest walks.
//   pair_match_kernel  one workgroup per (window, head): the window's kept bit rows, set from
//                      the index lists (row pitch odd, so that lanes reading one word of
//                      different rows hit different banks), written out as their complement
//                      for the linear branch (as mask_bits_kernel), and their pairwise
//                      overlaps in LDS; then wavefront 0 picks the pairs, one max-reduction
//                      over its lanes per pair, and writes each pair's union size where
//                      pair_order_kernel reads it (at the workgroup id that xcd_group_id gives
//                      the pair's slot).
constexpr int kMatchWin = 32;
constexpr int kMatchThreads = 256;
constexpr int kMatchPitch = kPairMaxWords + 1;

__global__ __launch_bounds__(kMatchThreads) void pair_match_kernel(const int32_t* __restrict__ idx, int nb,
                                                                  int nw, int topk, int npair, int xg,
                                                                  uint32_t* __restrict__ bits,
                                                                  int32_t* __restrict__ pairs,
                                                                  int32_t* __restrict__ size) {
  __shared__ uint32_t kb[kMatchWin * kMatchPitch];
  __shared__ int ov[kMatchWin][kMatchWin + 1];  // ov[a][b], a <= b: |K_a & K_b| (a = b: |K_a|)
  const int win = blockIdx.x, bh = blockIdx.y, tid = threadIdx.x;
  const int b0 = win * kMatchWin, nblk = min(kMatchWin, nb - b0);
  for (int e = tid; e < nblk * kMatchPitch; e += kMatchThreads) kb[e] = 0u;
  __syncthreads();
  // the window's index lists, eight loads in flight per thread before their LDS bit sets
  const int32_t* rows = idx + ((size_t)bh * nb + b0) * topk;
  const int nent = nblk * topk;
  for (int e0 = tid; e0 < nent; e0 += 8 * kMatchThreads) {
    int jv[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) jv[u] = e0 + u * kMatchThreads < nent ? rows[e0 + u * kMatchThreads] : -1;
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int e = e0 + u * kMatchThreads, j = jv[u];
      if (j >= 0 && j < nb) atomicOr(&kb[(e / topk) * kMatchPitch + j / 32], 1u << (j % 32));
    }
  }
  __syncthreads();
  // the complement rows (every block j < n_b not kept) for the linear branch's mask product
  for (int e = tid; e < nblk * nw; e += kMatchThreads) {
    const int i = e / nw, w = e % nw;
    const int valid = min(32, nb - 32 * w);
    const uint32_t all = valid == 32 ? 0xffffffffu : (1u << valid) - 1u;
    bits[((size_t)bh * nb + b0 + i) * nw + w] = all & ~kb[i * kMatchPitch + w];
  }
  for (int e = tid; e < kMatchWin * kMatchWin; e += kMatchThreads) {
    const int a = e / kMatchWin, b = e % kMatchWin;
    if (a <= b && b < nblk) {
      int o = 0;
#pragma unroll 4
      for (int w = 0; w < nw; ++w) o += __popc(kb[a * kMatchPitch + w] & kb[b * kMatchPitch + w]);
      ov[a][b] = o;
    }
  }
  __syncthreads();
  if (tid >= kWave) return;
  // lane (a, h) = (tid % 32, tid / 32) holds the half h of row a of the (symmetric) overlap
  // matrix in registers, partners b = 16 h + u; each round every lane of an unpaired a offers its
  // best unpaired partner as one key (overlap, then the lower index pair a' * 32 + b', a' < b',
  // first), and the wavefront's maximum key is the pair taken.  Lane r keeps pair r and all
  // pairs are written after the last round.
  constexpr int kHalf = kMatchWin / 2;
  const int a = tid % kMatchWin, h = tid / kMatchWin;
  int row[kHalf];
#pragma unroll
  for (int u = 0; u < kHalf; ++u) {
    const int b = kHalf * h + u;
    const int v = ov[min(a, b)][max(a, b)];
    row[u] = (a < nblk && b < nblk) ? v : 0;
  }
  uint32_t used = 0;  // wavefront-uniform
  int my_pa = 0, my_pb = 0, my_ov = 0;
  const int npw = nblk / 2;
  for (int r = 0; r < npw; ++r) {
    int key = -1;
    if (a < nblk && !((used >> a) & 1u)) {
#pragma unroll
      for (int u = 0; u < kHalf; ++u) {
        const int b = kHalf * h + u;
        if (b != a && b < nblk && !((used >> b) & 1u)) {
          const int pid = a < b ? a * kMatchWin + b : b * kMatchWin + a;
          key = max(key, (row[u] << 10) | (1023 - pid));
        }
      }
    }
    key = wave_max_int(key);
    const int pid = 1023 - (key & 1023), pa = pid / kMatchWin, pb = pid % kMatchWin;
    used |= (1u << pa) | (1u << pb);
    if (tid == r) {
      my_pa = pa;
      my_pb = pb;
      my_ov = key >> 10;
    }
  }
  int32_t* out = pairs + 2 * ((size_t)bh * npair + (size_t)win * kHalf);
  const int slot0 = win * kHalf;
  if (tid < npw) {
    out[2 * tid] = b0 + my_pa;
    out[2 * tid + 1] = b0 + my_pb;
    if (size) size[pair_id(xg, bh, slot0 + tid, npair)] = ov[my_pa][my_pa] + ov[my_pb][my_pb] - my_ov;
  } else if ((nblk & 1) && tid == npw) {  // the one block left (an odd window has nblk <= 31)
    const int left = __builtin_ctz(~used);
    out[2 * tid] = b0 + left;
    out[2 * tid + 1] = -1;
    if (size) size[pair_id(xg, bh, slot0 + tid, npair)] = ov[left][left];
  }
}

int pair_match_ints(const Dims& p) { return 2 * p.B * p.H * ((p.nb + 1) / 2); }

hipError_t launch_pair_match(const Dims& p, const int32_t* idx, uint32_t* bits, int32_t* pairs,
                             int32_t* size, bool unequal_heads, hipStream_t stream) {
  if (p.nb > kPairMaxWords * 32) return hipErrorInvalidValue;
  const dim3 grid((p.nb + kMatchWin - 1) / kMatchWin, p.B * p.H);
  pair_match_kernel<<<grid, kMatchThreads, 0, stream>>>(idx, p.nb, mask_words(p.nb), p.topk, (p.nb + 1) / 2,
                                                        pair_xg(unequal_heads), bits, pairs, size);
  return hipGetLastError();
}

hipError_t launch_pair_order(const Dims& p, const int32_t* size, int32_t* order, bool unequal_heads,
                             hipStream_t stream) {
  const int npair = (p.nb + 1) / 2, heads = p.B * p.H;
  const int xg = pair_xg(unequal_heads);
  const int smax = (npair + xg - 1) / xg;
  if (smax > kOrderMax) return hipErrorInvalidValue;
  const int groups = (heads + 8 / xg - 1) / (8 / xg);
  pair_order_kernel<<<dim3(8, groups), kOrderMax, 0, stream>>>(size, heads, npair, smax, xg, order);
  return hipGetLastError();
}

}  // namespace sla
