// sparse.hip - block-sparse softmax branch, the kept blocks' linear states, and the alpha
// combine, on gfx950.
//
// Sources: SLA2 Italian summary sections 1 and 2.A and Arabic summary sections 1 and 2.alef
// (sparse branch renormalised over the kept blocks; O = alpha O_s + (1 - alpha) O_l); SALAD
// section 2 (ReLU feature map of the linear branch, over the blocks the sparse branch leaves).
//
// One workgroup = one query block (64 rows) of one (batch, head), four wavefronts in two roles
// (the roles swap with the workgroup's parity so that co-resident workgroups pair a sparse and a
// state wavefront on a SIMD):
//   * two "sparse" wavefronts, 32 query rows each: S^T = K_j Q^T (v_mfma_f32_32x32x16_bf16, Q
//     in registers as the B operand, so each lane owns one query row and the row statistics stay
//     in-lane), online softmax in the log2 domain (the running maximum only moves when a row's
//     maximum grows by more than 2^8, so rescaling is rare), P rounded to bf16, row sums taken
//     from the bf16 P with v_dot2, and O_s^T += V_j^T P^T with the V operand read transposed
//     from LDS (ds_read_b64_tr_b16);
//   * two "state" wavefronts, each owning half of the d x d matrix
//     S_sel = sum over kept blocks of h_j = relu(K_j)^T V_j, accumulated from the same LDS
//     tiles (relu(K_j)^T and V_j both read transposed), i.e. the kept blocks' states recomputed
//     on chip instead of read from memory.
// K_j and V_j tiles are double-buffered in LDS (registers carry tile t+2 while tile t is used;
// one barrier per tile); the workgroup walks the router's ascending list.
// Epilogue: the state wavefronts form T = H - S_sel (H from the state kernel, fp32) split into
// bf16 hi + lo in LDS, and zeta = Z - sum_kept z_j; the sparse wavefronts compute
// num = relu(Q) T by MFMA, den = relu(q) . zeta, and O = alpha O_s / l + (1 - alpha) num / den
// (the linear part is 0 when nothing is unselected or den == 0), fp32 stores; rows past N are
// not stored.
#include <type_traits>

#include "sla_device.hpp"
#include "sla_launch.hpp"
#include "sla_tiles.hpp"

namespace sla {

namespace {

constexpr int kSparseThreads = 256;

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

template <class T, int D, bool FUSED>
__global__ __launch_bounds__(kSparseThreads, 2) void sparse_kernel(
    const T* __restrict__ Q, const T* __restrict__ K, const T* __restrict__ V,
    const int32_t* __restrict__ idx, const float* __restrict__ alpha,
    const __bf16* __restrict__ ht_hi, const __bf16* __restrict__ ht_lo,
    const float* __restrict__ Z, const float* __restrict__ zb, float* __restrict__ O, int N,
    int nb, int topk, float c_log2) {
  constexpr int NS = D / 16;       // MFMA k-steps over the head dim
  constexpr int NC = D / 32;       // 32-channel output tiles
  constexpr int RT = D / 64;       // 32-row tiles of S_sel per state wavefront
  constexpr int TILE = TileLayout<D>::ELEMS;
  // fp32 inputs keep K as bf16 hi + lo tiles so that S = K Q^T is about fp32-accurate
  // (Kh Qh + Kh Ql + Kl Qh); bf16 inputs are exact in one bf16 tile
  constexpr bool SPLIT = sizeof(T) == 4;
  constexpr int TILES = SPLIT ? 3 : 2;  // per buffer: K (hi), V, [K lo]
  // Two separate LDS arrays, one per tile buffer, so that the compiler can tell the buffer being
  // filled by direct-to-LDS loads from the one being read (with a single array it waits for the
  // in-flight loads before every read of the current tile).  After the loop they hold T^T hi
  // (buffer 0) and lo (buffer 1), each [D][D] in the tile row layout.
  static_assert(D * TileLayout<D>::PITCH <= TILES * TILE, "T^T must fit in one tile buffer");
  __shared__ __attribute__((aligned(16))) __bf16 lb0[TILES * TILE];
  __shared__ __attribute__((aligned(16))) __bf16 lb1[TILES * TILE];
  __shared__ float zeta[D];
  auto buf = [&](auto BUFC) -> __bf16* { return decltype(BUFC)::value ? lb1 : lb0; };

  const int tid = threadIdx.x;
  const int lane = tid % kWave, g = lane / 32;
  // wavefront-uniform as far as the compiler can tell, so role branches are scalar
  const int role = __builtin_amdgcn_readfirstlane(tid / kWave) ^ ((blockIdx.x & 1) ? 2 : 0);  // 0,1 sparse; 2,3 state
  const int item = xcd_remap(blockIdx.x, gridDim.x);
  const int bh = item / nb, qb = item % nb;
  const size_t hoff = (size_t)bh * N * D;
  const int32_t* sel = idx + ((size_t)bh * nb + qb) * topk;
  __bf16* t_hi = lb0;  // epilogue: T^T [c][c'] = H^T - S_sel^T (tile row layout), bf16 hi part
  __bf16* t_lo = lb1;  // and lo part

  // Tile staging shared by both roles: every thread moves its share of each tile.  bf16 tiles
  // with d = 128 and all 64 rows valid go HBM -> LDS directly (no registers), issued at the
  // start of the iteration that uses the other buffer; other tiles (fp32 inputs, d = 64, the
  // short last block) go through registers with zero fill, stored right away.  The state
  // role's z_j travels with the tile.  Both roles execute the same barriers: one after the
  // first tile, one per tile, one before the epilogue exchange.
  constexpr bool DIRECT = sizeof(T) == 2 && D == 128;
  const bool z_lane = FUSED && role >= 2 && (tid % 128) < D;
  float z_in = 0.f;        // z_j of the tile being staged (state role)
  int nv_next = kBlock;    // valid rows of the tile being staged
  float zacc = 0.f;        // state role: sum of z_j over the staged kept blocks
  auto stage = [&](int t, auto BUFC) {
    const int j = sel[t];
    const int nv = min(kBlock, N - j * kBlock);
    __bf16* dst = buf(BUFC);
    const T* ksrc = K + hoff + (size_t)j * kBlock * D;
    const T* vsrc = V + hoff + (size_t)j * kBlock * D;
    if (z_lane) z_in = zb[((size_t)bh * nb + j) * D + tid % 128];
    nv_next = nv;
    if constexpr (DIRECT) {
      // a short tile (the last block of the sequence) is clamped here and its tail rows are
      // zeroed after the loads land (zero_tail), so no register path sits in the loop
      if (nv == kBlock) {
        load_tile_direct<kSparseThreads>(ksrc, dst, tid);
        load_tile_direct<kSparseThreads>(vsrc, dst + TILE, tid);
      } else {
        load_tile_direct_clamped<kSparseThreads>(ksrc, dst, tid, nv);
        load_tile_direct_clamped<kSparseThreads>(vsrc, dst + TILE, tid, nv);
      }
    } else {
      TileLoader<T, D, kSparseThreads> lk, lv;
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
        zero_tile_rows<kSparseThreads>(buf(BUFC), tid, nv);
        zero_tile_rows<kSparseThreads>(buf(BUFC) + TILE, tid, nv);
        __syncthreads();
      }
    }
  };
  // LDS operand reads.  d = 128: per-lane address parts computed once and laundered through an
  // empty asm at the start of every tile (so the compiler re-derives the per-block addresses
  // with one v_xor each instead of holding dozens of them in registers across the loop); row
  // and buffer offsets are immediates.  d = 64: the padded layout's plain offsets.
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

  using B0 = std::integral_constant<int, 0>;
  using B1 = std::integral_constant<int, 1>;
  int nv_cur = kBlock;
  auto first = [&]() {
    if (topk > 0) {
      stage(0, B0{});
      zacc += z_in;
      nv_cur = nv_next;
      wait_vmem();
      __syncthreads();
      zero_tail(B0{}, nv_cur);
    }
  };
  // start staging tile t + 1 into the other buffer (last read in iteration t - 1)
  auto begin = [&](int t, auto BUFC) {
    launder();
    if (t + 1 < topk) stage(t + 1, std::integral_constant<int, 1 - decltype(BUFC)::value>{});
  };
  // after using tile t: publish tile t + 1
  auto end = [&](int t, auto BUFC) {
    nv_cur = nv_next;
    wait_vmem();
    __syncthreads();
    // z_j of tile t + 1 is added only now, after the explicit wait above: used earlier, the
    // compiler would wait for every in-flight tile load at that point
    __builtin_amdgcn_sched_barrier(0);
    if (t + 1 < topk) zacc += z_in;
    if (t + 1 < topk) zero_tail(std::integral_constant<int, 1 - decltype(BUFC)::value>{}, nv_cur);
  };
  // the kept tiles in pairs, so that each buffer index is a compile-time constant
  auto loop = [&](auto&& body) {
    for (int t = 0; t < topk; t += 2) {
      body(t, B0{});
      if (t + 1 < topk) body(t + 1, B1{});
    }
  };

  if (role < 2) {
    // ---------------- sparse role: 32 query rows ----------------
    // Q as the B operand of S^T = K Q^T: k-slot 8g + jj of step s <-> channel 16s + 8g + jj
    const int m = 32 * role + lane % 32;
    const int row = qb * kBlock + m;
    const bool row_ok = row < N;
    bf16x8 q[NS], ql[SPLIT ? NS : 1];
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      q[s] = row_ok ? load_row8<T>(Q + hoff + (size_t)row * D + 16 * s + 8 * g) : bf16x8{};
      if constexpr (SPLIT) ql[s] = row_ok ? load_row8_lo<T>(Q + hoff + (size_t)row * D + 16 * s + 8 * g) : bf16x8{};
    }
    f32x16 os[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c) os[c] = f32x16{};
    float mrun = -INFINITY, lsum = 0.f;

    first();
    loop([&](int t, auto BUFC) {
      const int nv = nv_cur;
      begin(t, BUFC);
      const __bf16* Ks = buf(BUFC);
      const __bf16* Vs = Ks + TILE;
      // K operands of both 32-key halves, issued together ahead of their MFMAs
      bf16x8 ka[2][NS];
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int k = 0; k < NS; ++k)
          ka[kt][k] = rd_row(Ks, 32 * kt, k);
      f32x16 s[2];
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        s[kt] = f32x16{};
#pragma unroll
        for (int k = 0; k < NS; ++k) {
          if constexpr (SPLIT) {
            s[kt] = mfma32(rd_row(Ks + 2 * TILE, 32 * kt, k), q[k], s[kt]);
            s[kt] = mfma32(ka[kt][k], ql[k], s[kt]);
          }
          s[kt] = mfma32(ka[kt][k], q[k], s[kt]);
        }
      }
      // V operands for PV: independent of P, so their LDS latency hides under the softmax
      bf16x8 va[NC][4];
#pragma unroll
      for (int c = 0; c < NC; ++c)
#pragma unroll
        for (int u = 0; u < 4; ++u) va[c][u] = rd_tr_v(Vs, 16 * u, 32 * c);
      // key of accumulator register i in half kt: 32kt + 8(i/4) + 4g + i%4
      if (nv < kBlock) {
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
      if (__ballot(mx > mrun + kRescaleSlack)) {
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
        for (int jj = 0; jj < 8; ++jj) pb[u][jj] = f2bf(fast_exp2(fmaf(s[u / 2][8 * (u % 2) + jj], c_log2, -mrun)));
        lsum = sum8(pb[u], lsum);
      }
      // O^T += V^T P^T ; MFMA u covers keys 16u .. 16u + 15
#pragma unroll
      for (int c = 0; c < NC; ++c)
#pragma unroll
        for (int u = 0; u < 4; ++u) os[c] = mfma32(va[c][u], pb[u], os[c]);
      end(t, BUFC);
    });
    __syncthreads();  // the state role has written T and zeta

    const float ltot = xor32_sum(lsum);
    const float inv_l = topk > 0 ? 1.f / ltot : 0.f;
    f32x16 num[NC];
    float inv_den = 0.f;
    if constexpr (FUSED) {
      // num^T[c][m] = sum_c' T^T[c][c'] relu(Q)[m][c'] (lo then hi part)
#pragma unroll
      for (int c = 0; c < NC; ++c) num[c] = f32x16{};
      float den = 0.f;
#pragma unroll
      for (int k = 0; k < NS; ++k) {
        const bf16x8 pq = relu8(q[k]);
#pragma unroll
        for (int c = 0; c < NC; ++c) {
          num[c] = mfma32(rd_row(t_lo, 32 * c, k), pq, num[c]);
          num[c] = mfma32(rd_row(t_hi, 32 * c, k), pq, num[c]);
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
    for (int c = 0; c < NC; ++c)
#pragma unroll
      for (int qd = 0; qd < 4; ++qd) {
        f32x4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float x = os[c][4 * qd + e] * ws;
          v[e] = FUSED ? fmaf(num[c][4 * qd + e], wl, x) : x;
        }
        *reinterpret_cast<f32x4*>(orow + 32 * c + 8 * qd + 4 * g) = v;
      }
  } else {
    // ---------------- state role: rows c' = cp0 .. cp0 + D/2 of S_sel ----------------
    const int cp0 = (role & 1) * (D / 2);
    const int st = tid % 128;  // index among the role's 128 threads (channel of z)
    f32x16 acc[RT][NC];
#pragma unroll
    for (int r = 0; r < RT; ++r)
#pragma unroll
      for (int c = 0; c < NC; ++c) acc[r][c] = f32x16{};

    first();
    loop([&](int t, auto BUFC) {
      begin(t, BUFC);
      if constexpr (FUSED) {
        const __bf16* Ks = buf(BUFC);
        const __bf16* Vs = Ks + TILE;
        // operands of key step ks + 1 are read while the MFMAs of step ks run
        bf16x8 a[2][RT], b[2][NC];
        auto rd = [&](int ks, int bsel) {
#pragma unroll
          for (int r = 0; r < RT; ++r) a[bsel][r] = rd_tr_s(Ks, 16 * ks, cp0 + 32 * r);
#pragma unroll
          for (int c = 0; c < NC; ++c) b[bsel][c] = rd_tr_s(Vs, 16 * ks, 32 * c);
        };
        rd(0, 0);
#pragma unroll
        for (int ks = 0; ks < kBlock / 16; ++ks) {
          if (ks + 1 < kBlock / 16) rd(ks + 1, (ks + 1) & 1);
#pragma unroll
          for (int r = 0; r < RT; ++r) {
            const bf16x8 ar = relu8(a[ks & 1][r]);
#pragma unroll
            for (int c = 0; c < NC; ++c) acc[r][c] = mfma32(ar, b[ks & 1][c], acc[r][c]);
          }
        }
      }
      end(t, BUFC);
    });
    if constexpr (FUSED) {
      const __bf16* hh = ht_hi + (size_t)bh * D * D;
      const __bf16* hl = ht_lo + (size_t)bh * D * D;
      // acc[r][c]: lane holds column c (V channel) = 32c + lane%32 and rows
      // c' = cp0 + 32r + 8(i/4) + 4g + i%4
#pragma unroll
      for (int r = 0; r < RT; ++r)
#pragma unroll
        for (int c = 0; c < NC; ++c) {
          const int cc = 32 * c + lane % 32;
#pragma unroll
          for (int qd = 0; qd < 4; ++qd) {
            const int cp = cp0 + 32 * r + 8 * qd + 4 * g;
            const bf16x4 h1 = *reinterpret_cast<const bf16x4*>(hh + (size_t)cc * D + cp);
            const bf16x4 h0 = *reinterpret_cast<const bf16x4*>(hl + (size_t)cc * D + cp);
            bf16x4 vh, vl;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const float tv = (bf2f(h1[e]) + bf2f(h0[e])) - acc[r][c][4 * qd + e];
              vh[e] = f2bf(tv);
              vl[e] = f2bf(tv - bf2f(vh[e]));
            }
            *reinterpret_cast<bf16x4*>(t_hi + TileLayout<D>::off(cc, cp)) = vh;
            *reinterpret_cast<bf16x4*>(t_lo + TileLayout<D>::off(cc, cp)) = vl;
          }
        }
      if (st < D) zeta[st] = Z[(size_t)bh * D + st] - zacc;
    }
    __syncthreads();
  }
}

template <class T, int D>
hipError_t launch_sparse_t(const Dims& p, const void* Q, const void* K, const void* V,
                           const int32_t* idx, const float* alpha, const __bf16* ht_hi,
                           const __bf16* ht_lo, const float* Z, const float* zb, float* O,
                           int fused, hipStream_t stream) {
  const int total = p.B * p.H * p.nb;
  const float c_log2 = 1.4426950408889634f / sqrtf((float)D);
  if (fused)
    sparse_kernel<T, D, true><<<total, kSparseThreads, 0, stream>>>(
        (const T*)Q, (const T*)K, (const T*)V, idx, alpha, ht_hi, ht_lo, Z, zb, O, p.N, p.nb,
        p.topk, c_log2);
  else
    sparse_kernel<T, D, false><<<total, kSparseThreads, 0, stream>>>(
        (const T*)Q, (const T*)K, (const T*)V, idx, alpha, ht_hi, ht_lo, Z, zb, O, p.N, p.nb,
        p.topk, c_log2);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_sparse(const Dims& p, const void* Q, const void* K, const void* V,
                         const int32_t* idx, const float* alpha, const __bf16* ht_hi,
                         const __bf16* ht_lo, const float* Z, const float* zb, float* O,
                         int fused, hipStream_t stream) {
  if (p.dtype == kBF16 && p.d == 128)
    return launch_sparse_t<__bf16, 128>(p, Q, K, V, idx, alpha, ht_hi, ht_lo, Z, zb, O, fused, stream);
  if (p.dtype == kBF16 && p.d == 64)
    return launch_sparse_t<__bf16, 64>(p, Q, K, V, idx, alpha, ht_hi, ht_lo, Z, zb, O, fused, stream);
  if (p.dtype == kF32 && p.d == 128)
    return launch_sparse_t<float, 128>(p, Q, K, V, idx, alpha, ht_hi, ht_lo, Z, zb, O, fused, stream);
  return launch_sparse_t<float, 64>(p, Q, K, V, idx, alpha, ht_hi, ht_lo, Z, zb, O, fused, stream);
}

}  // namespace sla
