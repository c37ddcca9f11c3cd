// bwd.hip - the backward of the SLA2 attention forward on gfx950 (the training path).
//
// SLA2 (Italian summary section 2, Arabic summary section 2): the model is fine-tuned with the
// sparse-linear attention in place; its QAT reading takes the backward on the unquantised
// values (Arabic summary section 2.jim).  Gradients of O = alpha O_s + (1 - alpha) O_l with
// respect to Q, K, V and alpha for given kept sets (the router's HardTop-k has none).  With
// dO_s = alpha dO, D_t = dO_s,t . O_s,t, g_t = (1 - alpha_t) dO_t / den_t, e_t = -g_t . O_l,t:
//   sparse  P = 2^(S c - lse2), dP = dO_s V^T, dS = P (dP - D), dQ += dS K / sqrt(d),
//           dK += dS^T Q / sqrt(d), dV += P^T dO_s
//   linear  dQ += (g A_i^T + e zeta_i) [q > 0], dA_i = relu(Q_i)^T G_i, dzeta_i = relu(Q_i)^T e_i,
//           dh_j = sum_{i: j unselected} dA_i, dz_j = likewise, dV += relu(K_j) dh_j,
//           dK += (V_j dh_j^T + dz_j) [k > 0]
//   dalpha_t = dO_t . (O_s,t - O_l,t).
//
//   prep_kernel      per (query block, head): dalpha, dO_s and G in bf16, D and e from them,
//                    dzeta_i (LDS reduction over the block's rows).
//   bits_t_kernel    the kept sets transposed: per key block j a bit row of the query blocks that
//                    keep it, and its complement (within n_b) for the mask GEMM.
//   (state_kernel mode 2 on (Q, G) gives every dA_i^T in the sliced bf16 layout of h_j^T;
//    tsel_kernel with the transposed complement gives every dh_j^T.)
//   dz_kernel        dz_j = sum over the query blocks leaving j unselected of dzeta_i.
//   bwd_dq_kernel    query-major, two query blocks per workgroup over the union of their kept
//                    lists (the forward's tile machinery): per tile S^T = K Q^T, P, dP^T =
//                    V dO_s^T, dS, dQ^T += K^T dS^T on bf16 MFMA; epilogue: the linear branch's
//                    dQ from T_i^T, zeta_i, G and e.
//   bwd_dkv_kernel   key-major, one key block per workgroup over the query blocks that keep it
//                    (Q and dO_s tiles, lse2 and D rows staged in LDS, double-buffered):
//                    wavefronts 0-1 accumulate dV^T += dO_s^T P for 32 keys each, wavefronts 2-3
//                    dK^T += Q^T dS (with dP = dO_s V^T), one 32-row query half of a tile at a
//                    time; epilogue: the linear branch's dV and dK from dh_j^T and dz_j.
// bf16 Q, K, V, dO with d = 128; gradients in fp32.
#include <type_traits>

#include "sla_device.hpp"
#include "sla_launch.hpp"
#include "sla_tiles.hpp"

namespace sla {

namespace {

constexpr int kBwdD = 128;
constexpr int kBwdThreads = 256;
constexpr int kBwdMaxWords = 64;  // n_b <= 2048

// ---------------------------------------------------------------------------------- prep

__global__ __launch_bounds__(kBwdThreads) void prep_kernel(
    const __bf16* __restrict__ Q, const __bf16* __restrict__ dO, const float* __restrict__ alpha,
    const float* __restrict__ Os, const float* __restrict__ Ol, const float* __restrict__ rden,
    int N, int nb, float* __restrict__ dalpha, __bf16* __restrict__ dOs, float* __restrict__ Dr,
    __bf16* __restrict__ G, float* __restrict__ e_out, float* __restrict__ dzeta) {
  constexpr int D = kBwdD;
  constexpr int TPR = D / 8;                 // threads per row: 8 channels (16 bytes of bf16) each
  constexpr int RPP = kBwdThreads / TPR;     // rows per pass
  __shared__ float red[RPP][D];
  const int tid = threadIdx.x;
  const int ch = (tid % TPR) * 8, rg = tid / TPR;
  const int i = blockIdx.x, bh = blockIdx.y;
  float zacc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) zacc[e] = 0.f;
  for (int pass = 0; pass < kBlock / RPP; ++pass) {
    const int row = i * kBlock + pass * RPP + rg;
    const bool ok = row < N;
    const size_t ro = ((size_t)bh * N + (ok ? row : 0)) * D + ch;
    const bf16x8 o8 = ok ? *reinterpret_cast<const bf16x8*>(dO + ro) : bf16x8{};
    const bf16x8 q8 = ok ? *reinterpret_cast<const bf16x8*>(Q + ro) : bf16x8{};
    const f32x4 os0 = ok ? *reinterpret_cast<const f32x4*>(Os + ro) : f32x4{};
    const f32x4 os1 = ok ? *reinterpret_cast<const f32x4*>(Os + ro + 4) : f32x4{};
    const f32x4 ol0 = ok ? *reinterpret_cast<const f32x4*>(Ol + ro) : f32x4{};
    const f32x4 ol1 = ok ? *reinterpret_cast<const f32x4*>(Ol + ro + 4) : f32x4{};
    const float a = ok ? alpha[(size_t)bh * N + row] : 0.f;
    const float rd = ok ? rden[(size_t)bh * N + row] : 0.f;
    float da = 0.f, dd = 0.f, ee = 0.f;
    bf16x8 s8, g8;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float o = bf2f(o8[e]);
      const float os = e < 4 ? os0[e] : os1[e - 4], ol = e < 4 ? ol0[e] : ol1[e - 4];
      da = fmaf(o, os - ol, da);
      s8[e] = f2bf(a * o);
      dd = fmaf(bf2f(s8[e]), os, dd);
      g8[e] = f2bf((1.f - a) * o * rd);
      ee = fmaf(bf2f(g8[e]), ol, ee);
    }
    if (ok) {
      *reinterpret_cast<bf16x8*>(dOs + ro) = s8;
      *reinterpret_cast<bf16x8*>(G + ro) = g8;
    }
    // row sums over the TPR consecutive lanes of the row
#pragma unroll
    for (int o = 1; o < TPR; o <<= 1) {
      da += __shfl_xor(da, o);
      dd += __shfl_xor(dd, o);
      ee += __shfl_xor(ee, o);
    }
    const float e = -ee;  // rows past N: 0
    if (ok && tid % TPR == 0) {
      dalpha[(size_t)bh * N + row] = da;
      Dr[(size_t)bh * N + row] = dd;
      e_out[(size_t)bh * N + row] = e;
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) zacc[k] = fmaf(e, fmaxf(bf2f(q8[k]), 0.f), zacc[k]);
  }
  // dzeta_i: the RPP row groups' partial sums through LDS, in a fixed order
#pragma unroll
  for (int k = 0; k < 8; ++k) red[rg][ch + k] = zacc[k];
  __syncthreads();
  if (tid < D) {
    float s = 0.f;
#pragma unroll
    for (int r = 0; r < RPP; ++r) s += red[r][tid];
    dzeta[((size_t)bh * nb + i) * D + tid] = s;
  }
}

// ---------------------------------------------------------------------------------- bits

// one workgroup per (32-bit word w of query blocks, head): the kept lists of query blocks 32 w ..
// 32 w + 31 are read once (coalesced) and each entry j sets bit b of key block j's word in LDS;
// then word w of every key block's kept row and of its complement (within n_b) is written out
__global__ __launch_bounds__(256) void bits_t_kernel(const int32_t* __restrict__ idx, int nb,
                                                     int topk, int nw, uint32_t* __restrict__ kept_t,
                                                     uint32_t* __restrict__ unsel_t) {
  __shared__ uint32_t bm[kBwdMaxWords * 32];
  const int bh = blockIdx.y, w = blockIdx.x, tid = threadIdx.x;
  for (int j = tid; j < nb; j += 256) bm[j] = 0u;
  __syncthreads();
  const int valid = min(32, nb - 32 * w);
  const int32_t* ib = idx + ((size_t)bh * nb + 32 * w) * topk;
  for (int q = tid; q < valid * topk; q += 256) {
    const int j = ib[q];
    if (j >= 0 && j < nb) atomicOr(&bm[j], 1u << (q / topk));
  }
  __syncthreads();
  const uint32_t all = valid == 32 ? 0xffffffffu : (1u << valid) - 1u;
  for (int j = tid; j < nb; j += 256) {
    const uint32_t kb = bm[j];
    kept_t[((size_t)bh * nb + j) * nw + w] = kb;
    unsel_t[((size_t)bh * nb + j) * nw + w] = all & ~kb;
  }
}

// ---------------------------------------------------------------------------------- dz

// the head's total of dzeta over its query blocks: a workgroup per (32 channels, head), 32 row
// groups x 8 lanes of 4 channels, reduced in a fixed order through LDS (deterministic)
__global__ __launch_bounds__(256) void dz_total_kernel(const float* __restrict__ dzeta, int nb,
                                                       float* __restrict__ tot) {
  constexpr int D = kBwdD;
  __shared__ float part[32][33];
  const int bh = blockIdx.y, tid = threadIdx.x;
  const int rg = tid / 8, cl = (tid % 8) * 4, c = blockIdx.x * 32 + cl;
  const float* zb = dzeta + (size_t)bh * nb * D;
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
  for (int i = rg; i < nb; i += 32) {
    const f32x4 a = *reinterpret_cast<const f32x4*>(zb + (size_t)i * D + c);
#pragma unroll
    for (int e = 0; e < 4; ++e) acc[e] += a[e];
  }
#pragma unroll
  for (int e = 0; e < 4; ++e) part[rg][cl + e] = acc[e];
  __syncthreads();
  if (tid < 32) {
    float t = 0.f;
#pragma unroll
    for (int r = 0; r < 32; ++r) t += part[r][tid];
    tot[(size_t)bh * D + blockIdx.x * 32 + tid] = t;
  }
}

// dz_j = sum over the query blocks leaving j unselected of dzeta_i, formed as the head's total
// minus the query blocks that keep j (about k of them instead of n_b - k).  A workgroup takes 16
// key blocks and stages their kept rows in LDS; thread (j = tid / 16, channels 8 (tid % 16) ..)
// walks its row and subtracts the kept query blocks in ascending order (deterministic), issuing
// the row loads four at a time
__global__ __launch_bounds__(256) void dz_kernel(const float* __restrict__ dzeta,
                                                 const float* __restrict__ tot,
                                                 const uint32_t* __restrict__ kept_t, int nb, int nw,
                                                 float* __restrict__ dz) {
  constexpr int D = kBwdD;
  __shared__ uint32_t kw[16][kBwdMaxWords];
  const int bh = blockIdx.y;
  const int tid = threadIdx.x;
  const int j0 = blockIdx.x * 16;
  for (int q = tid; q < 16 * nw; q += 256)
    kw[q / nw][q % nw] = j0 + q / nw < nb ? kept_t[((size_t)bh * nb + j0) * nw + q] : 0u;
  __syncthreads();
  const int jj = tid / 16, j = j0 + jj, c8 = (tid % 16) * 8;
  if (j >= nb) return;
  const float* zb = dzeta + (size_t)bh * nb * D + c8;
  const f32x4 t0 = *reinterpret_cast<const f32x4*>(tot + (size_t)bh * D + c8);
  const f32x4 t1 = *reinterpret_cast<const f32x4*>(tot + (size_t)bh * D + c8 + 4);
  float acc[8];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    acc[e] = t0[e];
    acc[4 + e] = t1[e];
  }
  int w = 0;
  uint32_t m = kw[jj][0];
  auto next = [&]() -> int {  // the next kept query block in ascending order, -1 past the end
    while (m == 0u) {
      if (++w >= nw) return -1;
      m = kw[jj][w];
    }
    const int i = 32 * w + __ffs(m) - 1;
    m &= m - 1u;
    return i;
  };
  for (;;) {
    int i[4];
    i[0] = next();
    if (i[0] < 0) break;
    i[1] = next();
    i[2] = next();
    i[3] = next();
    f32x4 a[4], b[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const float* r = zb + (size_t)(i[u] < 0 ? i[0] : i[u]) * D;
      a[u] = *reinterpret_cast<const f32x4*>(r);
      b[u] = *reinterpret_cast<const f32x4*>(r + 4);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (i[u] >= 0) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          acc[e] -= a[u][e];
          acc[4 + e] -= b[u][e];
        }
      }
  }
  float* o = dz + ((size_t)bh * nb + j) * D + c8;
  *reinterpret_cast<f32x4*>(o) = f32x4{acc[0], acc[1], acc[2], acc[3]};
  *reinterpret_cast<f32x4*>(o + 4) = f32x4{acc[4], acc[5], acc[6], acc[7]};
}

// ---------------------------------------------------------------------------------- dQ

__global__ __launch_bounds__(kBwdThreads, 2) void bwd_dq_kernel(
    const __bf16* __restrict__ Q, const __bf16* __restrict__ K, const __bf16* __restrict__ V,
    const int32_t* __restrict__ idx, const __bf16* __restrict__ dOs, const float* __restrict__ lse2,
    const float* __restrict__ Dr, const __bf16* __restrict__ G, const float* __restrict__ e_row,
    const __bf16* __restrict__ t_g, const float* __restrict__ Z, const float* __restrict__ zb,
    float* __restrict__ dQ, int N, int nb, int topk, float c_log2, float qscale) {
  constexpr int D = kBwdD;
  constexpr int NS = D / 16, NC = D / 32;
  constexpr int TILE = TileLayout<D>::ELEMS;
  __shared__ __attribute__((aligned(16))) __bf16 lb0[2 * TILE];
  __shared__ __attribute__((aligned(16))) __bf16 lb1[2 * TILE];
  __shared__ uint32_t bm[2][kBwdMaxWords];
  __shared__ int32_t ul[kBwdMaxWords * 32];
  __shared__ int32_t ucount;
  __shared__ float zeta[2][D];
  auto buf = [&](auto BUFC) -> __bf16* { return decltype(BUFC)::value ? lb1 : lb0; };

  const int tid = threadIdx.x;
  const int lane = tid % kWave, g = lane / 32;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int npair = (nb + 1) / 2;
  int bh, pr;
  if (!xcd_chunk_map(blockIdx.x, npair, &bh, &pr)) return;
  const int qb0 = 2 * pr;
  const bool has1 = qb0 + 1 < nb;
  const int blk = wave / 2;
  const size_t hoff = (size_t)bh * N * D;
  const int nw = (nb + 31) / 32;

  if (tid < 2 * kBwdMaxWords) bm[tid / kBwdMaxWords][tid % kBwdMaxWords] = 0u;
  __syncthreads();
  for (int t = tid; t < 2 * topk; t += kBwdThreads) {
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

  const int zb_blk = tid / D;
  const bool z_lane = tid < 2 * D;
  float z_in = 0.f, zacc = 0.f;
  int f_next = 0, nv_next = kBlock;
  auto stage = [&](int t, auto BUFC) {
    const int e = ul[t];
    const int j = e >> 2;
    const int nv = min(kBlock, N - j * kBlock);
    __bf16* dst = buf(BUFC);
    const __bf16* ksrc = K + hoff + (size_t)j * kBlock * D;
    const __bf16* vsrc = V + hoff + (size_t)j * kBlock * D;
    if (z_lane) z_in = zb[((size_t)bh * nb + j) * D + tid % D];
    f_next = e & 3;
    nv_next = nv;
    if (nv == kBlock) {
      load_tile_direct<kBwdThreads>(ksrc, dst, tid);
      load_tile_direct<kBwdThreads>(vsrc, dst + TILE, tid);
    } else {
      load_tile_direct_clamped<kBwdThreads>(ksrc, dst, tid, nv);
      load_tile_direct_clamped<kBwdThreads>(vsrc, dst + TILE, tid, nv);
    }
  };
  auto zero_tail = [&](auto BUFC, int nv) {
    if (nv < kBlock) {
      zero_tile_rows<kBwdThreads>(buf(BUFC), tid, nv);
      zero_tile_rows<kBwdThreads>(buf(BUFC) + TILE, tid, nv);
      __syncthreads();
    }
  };
  int ap_row = row_part(lane), ap_va = tr_part<4>(lane, 0), ap_vb = tr_part<4>(lane, 8);
  auto launder = [&]() { asm volatile("" : "+v"(ap_row), "+v"(ap_va), "+v"(ap_vb)); };
  auto rd_row = [&](const __bf16* tile, int R0, int k) -> bf16x8 {
    return lds_row16(tile, R0 * 256 + (ap_row ^ (32 * k)));
  };
  auto rd_tr = [&](const __bf16* tile, int row0, int col0) -> bf16x8 {
    return join_tr(lds_tr_at(tile, row0 * 256 + (ap_va ^ (2 * col0))),
                   lds_tr_at(tile, row0 * 256 + (ap_vb ^ (2 * col0))));
  };

  const int m = 32 * (wave % 2) + lane % 32;
  const int row = (qb0 + blk) * kBlock + m;
  const bool row_ok = row < N;
  const size_t rrow = hoff + (size_t)min(row, N - 1) * D;
  bf16x8 q[NS], dos[NS];
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    q[s] = row_ok ? *reinterpret_cast<const bf16x8*>(Q + rrow + 16 * s + 8 * g) : bf16x8{};
    dos[s] = row_ok ? *reinterpret_cast<const bf16x8*>(dOs + rrow + 16 * s + 8 * g) : bf16x8{};
  }
  const float l2 = row_ok ? lse2[(size_t)bh * N + row] : INFINITY;
  const float dr = row_ok ? Dr[(size_t)bh * N + row] : 0.f;
  f32x16 dq[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) dq[c] = f32x16{};

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
  // every path into the loop has waited for the operands loaded into registers above (else the
  // compiler waits for all memory traffic, the next tile's prefetch included, in every step)
  wait_vmem();
  auto step = [&](int t, auto BUFC) {
    constexpr int BUF = decltype(BUFC)::value;
    const int nv = nv_cur;
    launder();
    if (t + 1 < nu) stage(t + 1, std::integral_constant<int, 1 - BUF>{});
    if ((f_cur >> blk) & 1) {
      const __bf16* Ks = buf(BUFC);
      const __bf16* Vs = Ks + TILE;
      f32x16 s[2], dp[2];
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        s[kt] = f32x16{};
        dp[kt] = f32x16{};
      }
#pragma unroll
      for (int k = 0; k < NS; ++k)
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
          s[kt] = mfma32(rd_row(Ks, 32 * kt, k), q[k], s[kt]);
          dp[kt] = mfma32(rd_row(Vs, 32 * kt, k), dos[k], dp[kt]);
        }
      // dS = P (dP - D) in bf16; key of register i in half kt: 32 kt + 8 (i / 4) + 4 g + i % 4
      if (nv < kBlock) {  // the short last block (workgroup-uniform): keys past it get P = 0
        const int lim = nv - 4 * g;
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
          for (int i = 0; i < 16; ++i)
            if (32 * kt + 8 * (i / 4) + i % 4 >= lim) s[kt][i] = -INFINITY;
      }
      bf16x8 pb[4];
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) {
          const int kt = u / 2, i = 8 * (u % 2) + jj;
          pb[u][jj] = f2bf(fast_exp2(fmaf(s[kt][i], c_log2, -l2)) * (dp[kt][i] - dr));
        }
      // dQ^T += K^T dS^T: K read transposed (rows = keys in the k-order of pb)
#pragma unroll
      for (int c = 0; c < NC; ++c)
#pragma unroll
        for (int u = 0; u < 4; ++u) dq[c] = mfma32(rd_tr(Ks, 16 * u, 32 * c), pb[u], dq[c]);
    }
    nv_cur = nv_next;
    wait_vmem();
    __syncthreads();
    __builtin_amdgcn_sched_barrier(0);
    if (t + 1 < nu) {
      if (z_lane && ((f_next >> zb_blk) & 1)) zacc += z_in;
      f_cur = f_next;
      zero_tail(std::integral_constant<int, 1 - BUF>{}, nv_cur);
    }
  };
  {
    int t = 0;
    for (; t + 1 < nu; t += 2) {
      step(t, B0{});
      step(t + 1, B1{});
    }
    if (t < nu) step(t, B0{});
  }

  // ---- linear branch: T_i^T of block b into buffer b, zeta of each block ----
  const bool lin = topk < nb;
  if (lin) {
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      const __bf16* th = t_g + ((size_t)bh * nb + min(qb0 + b, nb - 1)) * D * D;
      __bf16* dst = b ? lb1 : lb0;
#pragma unroll
      for (int half = 0; half < D / kBlock; ++half)
        load_tile_direct<kBwdThreads>(th + half * kBlock * D, dst + half * kBlock * D, tid);
    }
    if (z_lane) zeta[zb_blk][tid % D] = Z[(size_t)bh * D + tid % D] - zacc;
    wait_vmem();
    __syncthreads();
    launder();
  }
  // dphi^T[c'][m] = sum_c A_i[c'][c] G[m][c] = sum_c T^T[c][c'] G[m][c]: the A operand is T^T
  // read transposed (k = c in the PV k-order), the B operand the lane's G row gathered in that
  // order (channels 16u + 4g + 0..3 and 16u + 8 + 4g + 0..3).  Every lane takes part (an MFMA
  // reads its operands from all 64 lanes): rows past N use zeros and store nothing.
  f32x16 dl[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) dl[c] = f32x16{};
  if (lin) {
    const __bf16* tt = blk ? lb1 : lb0;
    const __bf16* grow = G + rrow;
#pragma unroll
    for (int u = 0; u < NC * 2; ++u) {
      bf16x8 gb = bf16x8{};
      if (row_ok) {
        const bf16x4 g0 = *reinterpret_cast<const bf16x4*>(grow + 16 * u + 4 * g);
        const bf16x4 g1 = *reinterpret_cast<const bf16x4*>(grow + 16 * u + 8 + 4 * g);
        gb = bf16x8{g0[0], g0[1], g0[2], g0[3], g1[0], g1[1], g1[2], g1[3]};
      }
#pragma unroll
      for (int c = 0; c < NC; ++c) dl[c] = mfma32(rd_tr(tt, 16 * u, 32 * c), gb, dl[c]);
    }
  }
  if (!row_ok) return;
  const float er = e_row[(size_t)bh * N + row];
  // accumulator register 4 qd + e of tile c <-> channel 32 c + 8 qd + 4 g + e
  const __bf16* qrow = Q + hoff + (size_t)row * D;
  float* orow = dQ + hoff + (size_t)row * D;
#pragma unroll
  for (int c = 0; c < NC; ++c)
#pragma unroll
    for (int qd = 0; qd < 4; ++qd) {
      const int ch = 32 * c + 8 * qd + 4 * g;
      const bf16x4 qv = *reinterpret_cast<const bf16x4*>(qrow + ch);
      f32x4 v;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float lin_g = lin ? fmaf(er, zeta[blk][ch + e], dl[c][4 * qd + e]) : 0.f;
        v[e] = fmaf(dq[c][4 * qd + e], qscale, bf2f(qv[e]) > 0.f ? lin_g : 0.f);
      }
      *reinterpret_cast<f32x4*>(orow + ch) = v;
    }
}

// ---------------------------------------------------------------------------------- dK, dV

// One key block per workgroup.  Wavefronts 0-1 accumulate dV for keys 32 (w % 2) .. + 31 (the B
// operand, one key per lane), wavefronts 2-3 dK for the same keys; every tile is taken one
// 32-row query half at a time, so only one half's S, dP and P or dS are live at once.
__global__ __launch_bounds__(kBwdThreads, 2) void bwd_dkv_kernel(
    const __bf16* __restrict__ Q, const __bf16* __restrict__ K, const __bf16* __restrict__ V,
    const uint32_t* __restrict__ kept_t, const __bf16* __restrict__ dOs,
    const float* __restrict__ lse2, const float* __restrict__ Dr, const __bf16* __restrict__ dh_g,
    const float* __restrict__ dz, float* __restrict__ dK, float* __restrict__ dV, int N, int nb,
    int nw, float c_log2, float qscale) {
  constexpr int D = kBwdD;
  constexpr int NS = D / 16, NC = D / 32;
  constexpr int TILE = TileLayout<D>::ELEMS;
  // per buffer: Q_i tile, dO_s tile
  __shared__ __attribute__((aligned(16))) __bf16 lb0[2 * TILE];
  __shared__ __attribute__((aligned(16))) __bf16 lb1[2 * TILE];
  __shared__ __attribute__((aligned(16))) float rl[2][2][kBlock];  // [buffer][lse2 | D][row]
  __shared__ int32_t ql[kBwdMaxWords * 32];                          // query blocks keeping j
  __shared__ int32_t qcount;
  auto buf = [&](auto BUFC) -> __bf16* { return decltype(BUFC)::value ? lb1 : lb0; };

  const int tid = threadIdx.x;
  const int lane = tid % kWave, g = lane / 32;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  int bh, j;
  if (!xcd_chunk_map(blockIdx.x, nb, &bh, &j)) return;
  const size_t hoff = (size_t)bh * N * D;
  const bool dk_role = wave >= 2;  // wavefronts 0-1: dV, 2-3: dK
  const int kh = wave % 2;         // key half: keys 32 kh .. 32 kh + 31

  // ---- the query blocks that keep j, ascending ----
  if (wave == 0) {
    const uint32_t w = lane < nw ? kept_t[((size_t)bh * nb + j) * nw + lane] : 0u;
    const int cnt = __popc(w);
    int pos = cnt;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
      const int v = __shfl_up(pos, o);
      if (lane >= o) pos += v;
    }
    if (lane == kWave - 1) qcount = pos;
    pos -= cnt;
    for (uint32_t r = w; r; r &= r - 1) ql[pos++] = 32 * lane + __ffs(r) - 1;
  }
  __syncthreads();
  const int nq = qcount;

  int nv_next = kBlock;
  auto stage = [&](int t, auto BUFC) {
    constexpr int BUF = decltype(BUFC)::value;
    const int i = ql[t];
    const int nv = min(kBlock, N - i * kBlock);
    __bf16* dst = buf(BUFC);
    const __bf16* qsrc = Q + hoff + (size_t)i * kBlock * D;
    const __bf16* osrc = dOs + hoff + (size_t)i * kBlock * D;
    nv_next = nv;
    if (nv == kBlock) {
      load_tile_direct<kBwdThreads>(qsrc, dst, tid);
      load_tile_direct<kBwdThreads>(osrc, dst + TILE, tid);
    } else {
      load_tile_direct_clamped<kBwdThreads>(qsrc, dst, tid, nv);
      load_tile_direct_clamped<kBwdThreads>(osrc, dst + TILE, tid, nv);
    }
    if (tid < 2 * kBlock) {
      const int r = tid % kBlock, which = tid / kBlock;
      const bool ok = r < nv;
      const float v = ok ? (which ? Dr : lse2)[(size_t)bh * N + i * kBlock + min(r, nv - 1)] : 0.f;
      rl[BUF][which][r] = ok ? v : (which ? 0.f : INFINITY);
    }
  };
  auto zero_tail = [&](auto BUFC, int nv) {
    if (nv < kBlock) {
      zero_tile_rows<kBwdThreads>(buf(BUFC), tid, nv);
      zero_tile_rows<kBwdThreads>(buf(BUFC) + TILE, tid, nv);
      __syncthreads();
    }
  };
  int ap_row = row_part(lane), ap_va = tr_part<4>(lane, 0), ap_vb = tr_part<4>(lane, 8);
  auto launder = [&]() { asm volatile("" : "+v"(ap_row), "+v"(ap_va), "+v"(ap_vb)); };
  auto rd_row = [&](const __bf16* tile, int R0, int k) -> bf16x8 {
    return lds_row16(tile, R0 * 256 + (ap_row ^ (32 * k)));
  };
  auto rd_tr = [&](const __bf16* tile, int row0, int col0) -> bf16x8 {
    return join_tr(lds_tr_at(tile, row0 * 256 + (ap_va ^ (2 * col0))),
                   lds_tr_at(tile, row0 * 256 + (ap_vb ^ (2 * col0))));
  };

  // this wavefront's 32 keys as B operands (k-slot 8 g + jj of step s <-> channel 16 s + 8 g + jj)
  const int key = j * kBlock + 32 * kh + lane % 32;
  const bool key_ok = key < N;
  const size_t krow = hoff + (size_t)min(key, N - 1) * D;
  bf16x8 kr[NS], vr[NS];
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    kr[s] = key_ok ? *reinterpret_cast<const bf16x8*>(K + krow + 16 * s + 8 * g) : bf16x8{};
    vr[s] = (key_ok && dk_role) ? *reinterpret_cast<const bf16x8*>(V + krow + 16 * s + 8 * g) : bf16x8{};
  }
  f32x16 acc[NC];  // dV^T (wavefronts 0-1) or dK^T (2-3), rows = channels, column = this key
#pragma unroll
  for (int c = 0; c < NC; ++c) acc[c] = f32x16{};

  using B0 = std::integral_constant<int, 0>;
  using B1 = std::integral_constant<int, 1>;
  int nv_cur = kBlock;
  if (nq > 0) {
    stage(0, B0{});
    nv_cur = nv_next;
    wait_vmem();
    __syncthreads();
    zero_tail(B0{}, nv_cur);
  }
  // every path into the loop has waited for the operands loaded into registers above (else the
  // compiler waits for all memory traffic, the next tile's prefetch included, in every step)
  wait_vmem();
  auto step = [&](int t, auto BUFC) {
    constexpr int BUF = decltype(BUFC)::value;
    launder();
    if (t + 1 < nq) stage(t + 1, std::integral_constant<int, 1 - BUF>{});
    const __bf16* Qs = buf(BUFC);
    const __bf16* Os_t = Qs + TILE;
    const __bf16* At = dk_role ? Qs : Os_t;  // transposed A operand of the accumulation
#pragma unroll
    for (int qt = 0; qt < 2; ++qt) {
      // S[query][key] of query rows 32 qt .. (A = Q rows, B = this wavefront's keys); the dK
      // wavefronts also dP[query][key] = dO_s . V
      f32x16 s = f32x16{}, dp = f32x16{};
      if (dk_role) {
#pragma unroll
        for (int k = 0; k < NS; ++k) {
          s = mfma32(rd_row(Qs, 32 * qt, k), kr[k], s);
          dp = mfma32(rd_row(Os_t, 32 * qt, k), vr[k], dp);
        }
      } else {
#pragma unroll
        for (int k = 0; k < NS; ++k) s = mfma32(rd_row(Qs, 32 * qt, k), kr[k], s);
      }
      // register i <-> query 32 qt + 8 (i / 4) + 4 g + i % 4; lse2 and D of those rows
      const float* lr = rl[BUF][0] + 32 * qt;
      const float* dr = rl[BUF][1] + 32 * qt;
      bf16x8 pb[2];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const f32x4 l4 = *reinterpret_cast<const f32x4*>(lr + 8 * r + 4 * g);
        const f32x4 d4 = dk_role ? *reinterpret_cast<const f32x4*>(dr + 8 * r + 4 * g) : f32x4{};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int i = 4 * r + e;
          const float p = fast_exp2(fmaf(s[i], c_log2, -l4[e]));
          pb[i / 8][i % 8] = f2bf(dk_role ? p * (dp[i] - d4[e]) : p);
        }
      }
      // dV^T += dO_s^T P or dK^T += Q^T dS: the A operand read transposed from rows 32 qt + 16 u
#pragma unroll
      for (int c = 0; c < NC; ++c)
#pragma unroll
        for (int u = 0; u < 2; ++u) acc[c] = mfma32(rd_tr(At, 32 * qt + 16 * u, 32 * c), pb[u], acc[c]);
    }
    nv_cur = nv_next;
    wait_vmem();
    __syncthreads();
    __builtin_amdgcn_sched_barrier(0);
    if (t + 1 < nq) zero_tail(std::integral_constant<int, 1 - BUF>{}, nv_cur);
  };
  {
    int t = 0;
    for (; t + 1 < nq; t += 2) {
      step(t, B0{});
      step(t + 1, B1{});
    }
    if (t < nq) step(t, B0{});
  }

  // ---- linear branch: dh_j^T [c][c'] into buffer 0 (free since the last step's barrier).
  // Every lane takes part in the MFMAs below (they read operands from all 64 lanes); keys past
  // N hold zeros and store nothing ----
  {
    const __bf16* th = dh_g + ((size_t)bh * nb + j) * D * D;
#pragma unroll
    for (int half = 0; half < D / kBlock; ++half)
      load_tile_direct<kBwdThreads>(th + half * kBlock * D, lb0 + half * kBlock * D, tid);
  }
  wait_vmem();
  __syncthreads();
  launder();
  if (!dk_role) {
    // dV^T[c][key] += sum_c' dh^T[c][c'] relu(K)[key][c']: row reads of dh^T, relu(K) as B
#pragma unroll
    for (int k = 0; k < NS; ++k) {
      const bf16x8 pk = relu8(kr[k]);
#pragma unroll
      for (int c = 0; c < NC; ++c) acc[c] = mfma32(rd_row(lb0, 32 * c, k), pk, acc[c]);
    }
    if (!key_ok) return;
    float* o = dV + hoff + (size_t)key * D;
#pragma unroll
    for (int c = 0; c < NC; ++c)
#pragma unroll
      for (int qd = 0; qd < 4; ++qd)
        *reinterpret_cast<f32x4*>(o + 32 * c + 8 * qd + 4 * g) =
            f32x4{acc[c][4 * qd], acc[c][4 * qd + 1], acc[c][4 * qd + 2], acc[c][4 * qd + 3]};
  } else {
    // dK_lin^T[c'][key] = sum_c dh[c'][c] V[key][c]: dh^T read transposed (k = c in the PV
    // k-order) and the key's V row gathered in that order
    f32x16 dl[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c) dl[c] = f32x16{};
    const __bf16* vrow = V + krow;
#pragma unroll
    for (int u = 0; u < NC * 2; ++u) {
      bf16x8 vb = bf16x8{};
      if (key_ok) {
        const bf16x4 v0 = *reinterpret_cast<const bf16x4*>(vrow + 16 * u + 4 * g);
        const bf16x4 v1 = *reinterpret_cast<const bf16x4*>(vrow + 16 * u + 8 + 4 * g);
        vb = bf16x8{v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
      }
#pragma unroll
      for (int c = 0; c < NC; ++c) dl[c] = mfma32(rd_tr(lb0, 16 * u, 32 * c), vb, dl[c]);
    }
    if (!key_ok) return;
    const float* dzr = dz + ((size_t)bh * nb + j) * D;
    const __bf16* krw = K + hoff + (size_t)key * D;
    float* o = dK + hoff + (size_t)key * D;
#pragma unroll
    for (int c = 0; c < NC; ++c)
#pragma unroll
      for (int qd = 0; qd < 4; ++qd) {
        const int ch = 32 * c + 8 * qd + 4 * g;
        const bf16x4 kv = *reinterpret_cast<const bf16x4*>(krw + ch);
        f32x4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float lin_g = bf2f(kv[e]) > 0.f ? dl[c][4 * qd + e] + dzr[ch + e] : 0.f;
          v[e] = fmaf(acc[c][4 * qd + e], qscale, lin_g);
        }
        *reinterpret_cast<f32x4*>(o + ch) = v;
      }
  }
}

}  // namespace

hipError_t launch_bwd_prep(const Dims& p, const void* Q, const void* dO, const float* alpha,
                           const TrainRows& tr, float* dalpha, __bf16* dOs, float* Dr, __bf16* G,
                           float* e, float* dzeta, hipStream_t stream) {
  dim3 grid(p.nb, p.B * p.H);
  prep_kernel<<<grid, kBwdThreads, 0, stream>>>((const __bf16*)Q, (const __bf16*)dO, alpha, tr.Os,
                                                tr.Ol, tr.rden, p.N, p.nb, dalpha, dOs, Dr, G, e,
                                                dzeta);
  return hipGetLastError();
}

hipError_t launch_bits_t(const Dims& p, const int32_t* idx, uint32_t* kept_t, uint32_t* unsel_t,
                         hipStream_t stream) {
  const int nw = mask_words(p.nb);
  if (nw > kBwdMaxWords) return hipErrorInvalidValue;
  dim3 grid(nw, p.B * p.H);
  bits_t_kernel<<<grid, 256, 0, stream>>>(idx, p.nb, p.topk, nw, kept_t, unsel_t);
  return hipGetLastError();
}

hipError_t launch_bwd_dz(const Dims& p, const float* dzeta, const uint32_t* kept_t, float* tot,
                         float* dz, hipStream_t stream) {
  if (p.d != kBwdD) return hipErrorInvalidValue;
  dz_total_kernel<<<dim3(kBwdD / 32, p.B * p.H), 256, 0, stream>>>(dzeta, p.nb, tot);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  dim3 grid((p.nb + 15) / 16, p.B * p.H);
  dz_kernel<<<grid, 256, 0, stream>>>(dzeta, tot, kept_t, p.nb, mask_words(p.nb), dz);
  return hipGetLastError();
}

hipError_t launch_bwd_dq(const Dims& p, const void* Q, const void* K, const void* V,
                         const int32_t* idx, const __bf16* dOs, const float* lse2, const float* Dr,
                         const __bf16* G, const float* e, const __bf16* t_bf, const float* Z,
                         const float* zb, float* dQ, hipStream_t stream) {
  if (p.nb > kBwdMaxWords * 32) return hipErrorInvalidValue;
  const float qscale = 1.0f / sqrtf((float)kBwdD);
  const float c_log2 = 1.4426950408889634f * qscale;
  bwd_dq_kernel<<<xcd_chunk_grid(p.B * p.H, (p.nb + 1) / 2), kBwdThreads, 0, stream>>>(
      (const __bf16*)Q, (const __bf16*)K, (const __bf16*)V, idx, dOs, lse2, Dr, G, e, t_bf, Z, zb,
      dQ, p.N, p.nb, p.topk, c_log2, qscale);
  return hipGetLastError();
}

hipError_t launch_bwd_dkv(const Dims& p, const void* Q, const void* K, const void* V,
                          const uint32_t* kept_t, const __bf16* dOs, const float* lse2,
                          const float* Dr, const __bf16* dh, const float* dz, float* dK, float* dV,
                          hipStream_t stream) {
  if (p.nb > kBwdMaxWords * 32) return hipErrorInvalidValue;
  const float qscale = 1.0f / sqrtf((float)kBwdD);
  const float c_log2 = 1.4426950408889634f * qscale;
  bwd_dkv_kernel<<<xcd_chunk_grid(p.B * p.H, p.nb), kBwdThreads, 0, stream>>>(
      (const __bf16*)Q, (const __bf16*)K, (const __bf16*)V, kept_t, dOs, lse2, Dr, dh, dz, dK, dV,
      p.N, p.nb, mask_words(p.nb), c_log2, qscale);
  return hipGetLastError();
}

}  // namespace sla
