// fp8.hip - the quantised (QAT-forward) sparse branch on gfx950.
//
// SLA2 Italian summary section 2.C and Arabic summary section 2.jim: low-bit attention in the
// sparse branch only; the forward pass quantises Q, K, P and V.  Readings (the pages fix
// neither format nor granularity): OCP e4m3 (gfx950's native fp8), one absmax scale per
// (batch, head, 64-token block) for Q, K, V; P quantised per (query block x key block) tile
// with scale max(tile) / 448 over exp(S - rowmax) taken with the exact row maximum; the
// softmax denominator sums the unquantised exp(S - rowmax).
//
//   quantize_kernel   per (block, head): absmax -> inv = 448 / a, s = a / 448 (fp32, IEEE
//                     division), code = e4m3_rne(min(max(x * inv, -448), 448)).  Row-major
//                     codes, or (for V) a per-block transposed layout [d][64] whose key order
//                     matches the P operand of the PV MFMA.  The forwards use it for Q in the
//                     fused mode only (the state kernel writes the K and V codes, the
//                     mask-product kernel quantises its own query blocks, all with the helpers
//                     of sla_quant.hpp), and for everything under SLA_SEPARATE_QUANT=1.
//   sparse_fp8_kernel one workgroup per query block, four wavefronts in the two roles of the
//                     bf16 kernel.  Pass 1 over the kept blocks: the sparse wavefronts
//                     compute S = Q8 K8^T (v_mfma_scale_f32_32x32x64_f8f6f4, unit scales; K8
//                     fetched into registers one tile ahead) for each row's exact maximum,
//                     while the state wavefronts accumulate the kept blocks' relu(K_j)^T V_j
//                     from bf16 tiles (direct-to-LDS, as in the bf16 kernel).  Pass 2: K8 and
//                     V8^T tiles go straight into swizzled LDS; the sparse wavefronts recompute
//                     S, form P = exp(S - max), exchange the 64x64 tile maximum, quantise P and
//                     accumulate (P8 V8) sP sV by fp8 MFMA.  Epilogue and combine as in the
//                     bf16 kernel.
//
// INT8 (the other low-bit format the SLA2 summaries name for the sparse branch): the quantiser
// and the two-query-block kernel are templated on the code format.  int8 codes are symmetric
// (+-127, ties to even) with scale a / 127 per block, P's tile scale is max(tile) / 127, and the
// products run on v_mfma_i32_32x32x32_i8 (each 32-byte fp8 operand chunk is two 16-byte int8
// operands; int32 accumulation is exact: |S| <= 128 * 127^2, |PV| <= 64 * 127^2 < 2^24, so the
// conversion to fp32 is exact too).  P's codes come from one fma with 1.5 * 2^23, which leaves
// round-half-even(P / sP) in the low byte of the float.
#include <type_traits>

#include "sla_device.hpp"
#include "sla_launch.hpp"
#include "sla_tiles.hpp"
#include "sla_quant.hpp"

namespace sla {

namespace {


__device__ __forceinline__ f32x16 mfma_f8(i32x8 a, i32x8 b, f32x16 c) {
  // formats 0/0 = e4m3 for both operands; scale exponents 127 = 2^0
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}
typedef int i32x16 __attribute__((ext_vector_type(16)));
// 64-deep int8 product of two 32-byte operand chunks: two v_mfma_i32_32x32x32_i8 over the
// halves (A and B use the same byte order, so the k-slot assignment inside the halves is free)
__device__ __forceinline__ i32x16 mfma_i8x64(i32x8 a, i32x8 b, i32x16 c) {
  c = __builtin_amdgcn_mfma_i32_32x32x32_i8(i32x4{a[0], a[1], a[2], a[3]}, i32x4{b[0], b[1], b[2], b[3]}, c, 0, 0, 0);
  return __builtin_amdgcn_mfma_i32_32x32x32_i8(i32x4{a[4], a[5], a[6], a[7]}, i32x4{b[4], b[5], b[6], b[7]}, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 i2f16(i32x16 v) {
  f32x16 r;
#pragma unroll
  for (int i = 0; i < 16; ++i) r[i] = (float)v[i];
  return r;
}
// int8 codes of p * qs for 4 non-negative p with p * qs below 127.5: fma(p, qs, 1.5 * 2^23)
// rounds the exact product once to an integer (ties to even) held in the float's low byte
__device__ __forceinline__ u32 cvt4_u7(float a, float b, float c, float d, float qs) {
  constexpr float kMagic = 12582912.f;
  const u32 x = __float_as_uint(fmaf(a, qs, kMagic)), y = __float_as_uint(fmaf(b, qs, kMagic));
  const u32 z = __float_as_uint(fmaf(c, qs, kMagic)), w = __float_as_uint(fmaf(d, qs, kMagic));
  return (x & 0xffu) | ((y & 0xffu) << 8) | ((z & 0xffu) << 16) | (w << 24);
}

template <int D, bool TRANSPOSED, int FMT>
__global__ __launch_bounds__(256) void quantize_kernel(const __bf16* __restrict__ X, int N,
                                                       int nb, uint8_t* __restrict__ codes,
                                                       float* __restrict__ scales) {
  __shared__ float wmax[4];
  __shared__ __attribute__((aligned(16))) uint8_t tl[TRANSPOSED ? D * kBlock : 16];
  const int tid = threadIdx.x, lane = tid % kWave, w = tid / kWave;
  const int t = blockIdx.x, bh = blockIdx.y;
  const int row0 = t * kBlock;
  const int cnt = min(kBlock, N - row0);
  constexpr int CPR = D / 8;                  // 16-byte chunks per row
  constexpr int PER = kBlock * CPR / 256;     // chunks per thread
  const __bf16* Xb = X + ((size_t)bh * N + row0) * D;
  i32x4 v[PER];
#pragma unroll
  for (int u = 0; u < PER; ++u) {
    const int q = tid + u * 256, r = q / CPR, ch = q % CPR;
    v[u] = r < cnt ? ld16(Xb + (size_t)r * D + ch * 8) : i32x4{0, 0, 0, 0};
  }
  float amax = wave_max(qz_local_amax(v));
  if (lane == 0) wmax[w] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]));
  const float inv = qz_inv<FMT>(amax);
  if (tid == 0) scales[(size_t)bh * nb + t] = qz_scale<FMT>(amax);
#pragma unroll
  for (int u = 0; u < PER; ++u) {
    const int q = tid + u * 256, r = q / CPR, ch = q % CPR;
    if constexpr (!TRANSPOSED) {
      if (r >= cnt) continue;  // past N: no such row in the output
      *reinterpret_cast<uint2*>(codes + ((size_t)bh * N + row0 + r) * D + ch * 8) = qz_row_codes<FMT>(v[u], inv);
    } else {
      // [c][pos(r)] staged in LDS (keys past N get code 0: their P8 is 0 as well)
      qz_tr_codes<FMT>(v[u], inv, tl, r, ch);
    }
  }
  if constexpr (TRANSPOSED) {
    __syncthreads();
    qz_tr_flush<D, 256>(tl, codes + ((size_t)bh * nb + t) * D * kBlock, tid);  // [bh][t][c][pos]
  }
}

constexpr int kF8Threads = 256;

// LDS layouts of the pass-2 tiles:
//   K8  [64 keys][128 B]: 16-byte unit u of row r at unit u ^ ((r >> 1) & 7)
//   V8t [128 channels][64 B]: 16-byte unit u of row c at unit u ^ ((c >> 2) & 3)
// so that 16 consecutive rows reading one unit hit 16 distinct 16-byte bank groups.
__device__ __forceinline__ int k8_off(int r, int b) { return r * 128 + ((((b >> 4) ^ ((r >> 1) & 7))) << 4) + (b & 15); }
__device__ __forceinline__ int v8_off(int c, int b) { return c * 64 + ((((b >> 4) ^ ((c >> 2) & 3))) << 4) + (b & 15); }

__device__ __forceinline__ i32x8 join8(i32x4 a, i32x4 b) {
  return i32x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}

template <int D>
__global__ __launch_bounds__(kF8Threads, 2) void sparse_fp8_kernel(
    const __bf16* __restrict__ Q, const __bf16* __restrict__ K, const __bf16* __restrict__ V,
    const uint8_t* __restrict__ q8, const uint8_t* __restrict__ k8,
    const uint8_t* __restrict__ v8t, const float* __restrict__ sq,
    const float* __restrict__ sk, const float* __restrict__ sv,
    const int32_t* __restrict__ idx, const float* __restrict__ alpha,
    const __bf16* __restrict__ ht_hi, const __bf16* __restrict__ ht_lo,
    const float* __restrict__ Z, const float* __restrict__ zb, float* __restrict__ O, int N,
    int nb, int topk, float c_log2) {
  static_assert(D == 128, "the fp8 kernel is compiled for d = 128");
  constexpr int NS = D / 16, NC = D / 32, RT = D / 64, N8 = D / 64;
  constexpr int TILE = TileLayout<D>::ELEMS;  // bf16 elements of a K or V tile
  constexpr int K8B = kBlock * D;             // bytes of a K8 tile
  // One LDS array per buffer, so that the compiler can tell the buffer being filled by
  // direct-to-LDS loads from the one being read.  Pass 1: bf16 K, V tiles; pass 2: K8 and V8^T
  // tiles; afterwards T^T hi (buffer 0) and lo (buffer 1), each [D][D] in the tile row layout.
  __shared__ __attribute__((aligned(16))) __bf16 lb0[2 * TILE];
  __shared__ __attribute__((aligned(16))) __bf16 lb1[2 * TILE];
  __shared__ float zeta[D];
  __shared__ float tmax_x[2];
  auto buf = [&](auto BUFC) -> __bf16* { return decltype(BUFC)::value ? lb1 : lb0; };
  auto buf8 = [&](auto BUFC) -> uint8_t* { return reinterpret_cast<uint8_t*>(buf(BUFC)); };
  using B0 = std::integral_constant<int, 0>;
  using B1 = std::integral_constant<int, 1>;

  const int tid = threadIdx.x;
  const int lane = tid % kWave, g = lane / 32;
  const int w = __builtin_amdgcn_readfirstlane(tid / kWave);  // wavefront-uniform (scalar branches)
  const int role = w ^ ((blockIdx.x & 1) ? 2 : 0);  // 0,1 sparse; 2,3 state
  const int item = xcd_remap(blockIdx.x, gridDim.x);
  const int bh = item / nb, qb = item % nb;
  const size_t hoff = (size_t)bh * N * D;
  const int32_t* sel = idx + ((size_t)bh * nb + qb) * topk;
  const float sqi = sq[(size_t)bh * nb + qb];
  __bf16* t_hi = lb0;
  __bf16* t_lo = lb1;

  // the kept tiles in pairs, so that each buffer index is a compile-time constant
  auto loop = [&](auto&& body) {
    for (int t = 0; t < topk; t += 2) {
      body(t, B0{});
      if (t + 1 < topk) body(t + 1, B1{});
    }
  };
  // ---- pass 1 staging: bf16 K, V tiles (state role's linear states); a short tile is clamped
  // and its tail rows zeroed once the loads have landed ----
  const bool z_lane = role >= 2 && (tid % 128) < D;
  float z_in = 0.f, zacc = 0.f;
  int nv_next = kBlock;
  auto stage1 = [&](int t, auto BUFC) {
    const int j = sel[t];
    const int nv = min(kBlock, N - j * kBlock);
    __bf16* dst = buf(BUFC);
    const __bf16* ksrc = K + hoff + (size_t)j * kBlock * D;
    const __bf16* vsrc = V + hoff + (size_t)j * kBlock * D;
    if (z_lane) z_in = zb[((size_t)bh * nb + j) * D + tid % 128];
    nv_next = nv;
    if (nv == kBlock) {
      load_tile_direct<kF8Threads>(ksrc, dst, tid);
      load_tile_direct<kF8Threads>(vsrc, dst + TILE, tid);
    } else {
      load_tile_direct_clamped<kF8Threads>(ksrc, dst, tid, nv);
      load_tile_direct_clamped<kF8Threads>(vsrc, dst + TILE, tid, nv);
    }
  };
  auto publish1 = [&](int t, auto NEXT) {  // after the staged loads of tile t (if any) landed
    wait_vmem();
    __syncthreads();
    __builtin_amdgcn_sched_barrier(0);
    if (t < topk) {
      zacc += z_in;
      if (nv_next < kBlock) {
        zero_tile_rows<kF8Threads>(buf(NEXT), tid, nv_next);
        zero_tile_rows<kF8Threads>(buf(NEXT) + TILE, tid, nv_next);
        __syncthreads();
      }
    }
  };
  // ---- pass 2 staging: K8 and V8^T tiles (sparse role), straight into the swizzled layouts ----
  auto stage2 = [&](int t, auto BUFC) {
    const int j = sel[t];
    const int nv = min(kBlock, N - j * kBlock);
    uint8_t* dst = buf8(BUFC);
    const uint8_t* ksrc = k8 + hoff + (size_t)j * kBlock * D;
    const uint8_t* vsrc = v8t + ((size_t)bh * nb + j) * D * kBlock;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int r0 = 8 * (2 * w + u);  // 8 K8 rows of 128 B per wave load
      const int r = r0 + lane / 8;
      const int unit = (lane % 8) ^ ((r >> 1) & 7);
      load_lds16(ksrc + (size_t)min(r, nv - 1) * D + unit * 16, dst + r0 * 128);
      const int c0 = 16 * (2 * w + u);  // 16 V8^T rows of 64 B per wave load
      const int c = c0 + lane / 4;
      const int vunit = (lane % 4) ^ ((c >> 2) & 3);
      load_lds16(vsrc + (size_t)c * kBlock + vunit * 16, dst + K8B + c0 * 64);
    }
  };

  if (role < 2) {
    // ================= sparse role: 32 query rows =================
    const int m = 32 * role + lane % 32;
    const int row = qb * kBlock + m;
    const bool row_ok = row < N;
    const bool rows_all_ok = __ballot(!row_ok) == 0;  // every row of this wavefront exists
    i32x8 qf[N8];  // e4m3 Q as the B operand: k-slot 32g + b of step s <-> channel 64s + 32g + b
#pragma unroll
    for (int s = 0; s < N8; ++s) {
      if (row_ok) {
        const i32x4* p = reinterpret_cast<const i32x4*>(q8 + hoff + (size_t)row * D + 64 * s + 32 * g);
        qf[s] = join8(p[0], p[1]);
      } else {
        qf[s] = i32x8{};
      }
    }
    // pass 1: exact row maximum of S (log2 units); K8 operands come straight from memory, one
    // tile ahead (rows past a short block's end re-read its last row: those keys are masked)
    auto k8_regs = [&](int t, i32x8 (&kr)[2][N8]) {
      const int j = sel[t];
      const int nv = min(kBlock, N - j * kBlock);
      const uint8_t* src = k8 + hoff + (size_t)j * kBlock * D;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int st = 0; st < N8; ++st) {
          const i32x4* p = reinterpret_cast<const i32x4*>(src + (size_t)min(32 * kt + lane % 32, nv - 1) * D + 64 * st + 32 * g);
          kr[kt][st] = join8(p[0], p[1]);
        }
    };
    float mrow = -INFINITY;
    i32x8 kr[2][2][N8];
    if (topk > 0) {
      stage1(0, B0{});
      k8_regs(0, kr[0]);
      publish1(0, B0{});
    }
    loop([&](int t, auto BUFC) {
      constexpr int BUF = decltype(BUFC)::value;
      using NEXT = std::integral_constant<int, 1 - BUF>;
      if (t + 1 < topk) {
        stage1(t + 1, NEXT{});
        k8_regs(t + 1, kr[1 - BUF]);
      }
      const int j = sel[t];
      const int nv = min(kBlock, N - __builtin_amdgcn_readfirstlane(j) * kBlock);
      const float sc = sqi * sk[(size_t)bh * nb + j] * c_log2;
      const int lim = nv - 4 * g;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        f32x16 s = f32x16{};
#pragma unroll
        for (int st = 0; st < N8; ++st) s = mfma_f8(kr[BUF][kt][st], qf[st], s);
        if (nv == kBlock) {  // a full tile: no key mask; sc > 0 scales the maximum once
          float mx = s[0];
#pragma unroll
          for (int i = 1; i < 16; ++i) mx = fmaxf(mx, s[i]);
          mrow = fmaxf(mrow, mx * sc);
        } else {
#pragma unroll
          for (int i = 0; i < 16; ++i)
            if (32 * kt + 8 * (i / 4) + i % 4 < lim) mrow = fmaxf(mrow, s[i] * sc);
        }
      }
      publish1(t + 1, NEXT{});
    });
    mrow = xor32_max(mrow);

    // pass 2: P with the exact maximum, 64x64 tile maximum across both wavefronts, fp8 PV
    f32x16 os[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c) os[c] = f32x16{};
    float lsum = 0.f;
    if (topk > 0) {
      stage2(0, B0{});
      wait_vmem();
      __syncthreads();
    }
    loop([&](int t, auto BUFC) {
      constexpr int BUF = decltype(BUFC)::value;
      if (t + 1 < topk) stage2(t + 1, std::integral_constant<int, 1 - BUF>{});
      const int j = sel[t];
      const int nv = min(kBlock, N - j * kBlock);
      const uint8_t* ks = buf8(BUFC);
      const uint8_t* vs = ks + K8B;
      const float sc = sqi * sk[(size_t)bh * nb + j] * c_log2;
      const int lim = row_ok ? nv - 4 * g : 0;
      float p[2][16];
      float pmax = 0.f;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        f32x16 s = f32x16{};
#pragma unroll
        for (int st = 0; st < N8; ++st) {
          const int r = 32 * kt + lane % 32;
          const i32x4 a0 = *reinterpret_cast<const i32x4*>(ks + k8_off(r, 64 * st + 32 * g));
          const i32x4 a1 = *reinterpret_cast<const i32x4*>(ks + k8_off(r, 64 * st + 32 * g + 16));
          s = mfma_f8(join8(a0, a1), qf[st], s);
        }
        if (rows_all_ok && nv == kBlock) {  // wavefront-uniform: no key or row mask
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            p[kt][i] = fast_exp2(fmaf(s[i], sc, -mrow));
            lsum += p[kt][i];
            pmax = fmaxf(pmax, p[kt][i]);
          }
        } else {
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            p[kt][i] = 32 * kt + 8 * (i / 4) + i % 4 < lim ? fast_exp2(fmaf(s[i], sc, -mrow)) : 0.f;
            lsum += p[kt][i];
            pmax = fmaxf(pmax, p[kt][i]);
          }
        }
      }
      pmax = wave_max(pmax);
      if (lane == 0) tmax_x[role] = pmax;
      // V8^T operands (independent of the tile maximum)
      i32x8 va[NC];
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        const int cr = 32 * c + lane % 32;
        va[c] = join8(*reinterpret_cast<const i32x4*>(vs + v8_off(cr, 32 * g)),
                      *reinterpret_cast<const i32x4*>(vs + v8_off(cr, 32 * g + 16)));
      }
      __syncthreads();
      const float tmax = fmaxf(tmax_x[0], tmax_x[1]);
      const float qs = tmax > 0.f ? kE4M3Max / tmax : 0.f;  // an all-underflow tile adds 0
      // P8 as the B operand: slot 16kt + i <-> key 32kt + 8(i/4) + 4g + i%4
      i32x8 pf;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int qd = 0; qd < 4; ++qd)
          pf[4 * kt + qd] = (int)cvt4_e4m3(sat(p[kt][4 * qd] * qs), sat(p[kt][4 * qd + 1] * qs),
                                           sat(p[kt][4 * qd + 2] * qs), sat(p[kt][4 * qd + 3] * qs));
      const float pv_scale = (tmax / kE4M3Max) * sv[(size_t)bh * nb + j];
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        const f32x16 tmp = mfma_f8(va[c], pf, f32x16{});
        os[c] += tmp * pv_scale;
      }
      wait_vmem();
      __syncthreads();
    });
    // this row of Q for the linear numerator, read before the barrier so that the loads are in
    // flight while it waits (unconditional, from a clamped row: a load under a branch makes the
    // compiler wait for it on the spot)
    bf16x8 qv[NS];
    {
      const __bf16* qr = Q + hoff + (size_t)min(row, N - 1) * D + 8 * g;
#pragma unroll
      for (int k = 0; k < NS; ++k) qv[k] = *reinterpret_cast<const bf16x8*>(qr + 16 * k);
    }
    __syncthreads();  // the state role has written T and zeta

    // epilogue (as in the bf16 kernel): linear numerator relu(Q) T, denominator, combine
    const float ltot = xor32_sum(lsum);
    const float inv_l = topk > 0 ? 1.f / ltot : 0.f;
    f32x16 num[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c) num[c] = f32x16{};
    float den = 0.f;
#pragma unroll
    for (int k = 0; k < NS; ++k) {
      const bf16x8 pq = relu8(row_ok ? qv[k] : bf16x8{});
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        const int off = TileLayout<D>::off(32 * c + lane % 32, 16 * k + 8 * g);
        num[c] = mfma32(*reinterpret_cast<const bf16x8*>(t_lo + off), pq, num[c]);
        num[c] = mfma32(*reinterpret_cast<const bf16x8*>(t_hi + off), pq, num[c]);
      }
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) den += bf2f(pq[jj]) * zeta[16 * k + 8 * g + jj];
    }
    den = xor32_sum(den);
    const float inv_den = (topk < nb && den != 0.f) ? 1.f / den : 0.f;
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
        for (int e = 0; e < 4; ++e) v[e] = fmaf(num[c][4 * qd + e], wl, os[c][4 * qd + e] * ws);
        *reinterpret_cast<f32x4*>(orow + 32 * c + 8 * qd + 4 * g) = v;
      }
  } else {
    // ================= state role: rows c' = cp0 .. cp0 + D/2 of S_sel (pass 1) =================
    const int cp0 = (role & 1) * (D / 2);
    const int st = tid % 128;
    f32x16 acc[RT][NC];
#pragma unroll
    for (int r = 0; r < RT; ++r)
#pragma unroll
      for (int c = 0; c < NC; ++c) acc[r][c] = f32x16{};
    if (topk > 0) {
      stage1(0, B0{});
      publish1(0, B0{});
    }
    loop([&](int t, auto BUFC) {
      constexpr int BUF = decltype(BUFC)::value;
      using NEXT = std::integral_constant<int, 1 - BUF>;
      if (t + 1 < topk) stage1(t + 1, NEXT{});
      const __bf16* Ks = buf(BUFC);
      const __bf16* Vs = Ks + TILE;
      bf16x8 a[2][RT], b[2][NC];
      auto rd = [&](int ks, int bsel) {
#pragma unroll
        for (int r = 0; r < RT; ++r) a[bsel][r] = tr_operand<D, 8, 4>(Ks, 16 * ks, cp0 + 32 * r, lane);
#pragma unroll
        for (int c = 0; c < NC; ++c) b[bsel][c] = tr_operand<D, 8, 4>(Vs, 16 * ks, 32 * c, lane);
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
      publish1(t + 1, NEXT{});
    });
    // pass 2: only the tile staging and the barriers (two per tile)
    if (topk > 0) {
      stage2(0, B0{});
      wait_vmem();
      __syncthreads();
    }
    loop([&](int t, auto BUFC) {
      if (t + 1 < topk) stage2(t + 1, std::integral_constant<int, 1 - decltype(BUFC)::value>{});
      __syncthreads();
      wait_vmem();
      __syncthreads();
    });
    // T = H - S_sel (bf16 hi + lo) and zeta = Z - sum_kept z_j for the sparse role
    const __bf16* hh = ht_hi + (size_t)bh * D * D;
    const __bf16* hl = ht_lo + (size_t)bh * D * D;
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
    __syncthreads();
  }
}

// The quantised sparse branch for two query blocks per workgroup, with the linear branch's
// T_i = sum of the unselected blocks' states taken from memory (mask-product mode).  Wavefront w
// takes rows 32 (w % 2) .. + 31 of query block 2p + w / 2.  Q's codes come from the stand-alone
// quantiser (q8) or, q8 null, from this workgroup, which quantises its two query blocks itself.
//   Pass 1 (no LDS, no barrier): each wavefront walks its own block's kept list with its K8
//   operands read straight from memory one tile ahead, S = Q8 K8^T, each row's exact maximum;
//   z_j of the kept blocks summed on the way.
//   Pass 2: the workgroup walks the ascending union of the two lists and stages each K8 and V8^T
//   tile into LDS once for both blocks (K one step ahead of V); per tile t a wavefront whose
//   block kept it forms S and, per row, log2 of its largest P^ = 2^(S sc - m) in the tile (no
//   exponential: max(S) sc - m), whose max over its 32 rows meets the partner wavefront's in LDS
//   at the step's barrier.  In step t + 1, with e = log2 max(tile), each P code comes from one
//   exponential, code(2^(S sc - m + log2 448 - e)) = code(P^ 448 / max), and (P8 V8) sP sV is
//   accumulated by fp8 MFMA with sP = 2^e / 448: one barrier per tile.  The denominator sums the
//   unquantised P^ = y sP.
template <int D, int FMT>
__global__ __launch_bounds__(kF8Threads, 2) void pair8_kernel(
    const __bf16* __restrict__ Q, const uint8_t* __restrict__ q8,
    const uint8_t* __restrict__ k8, const uint8_t* __restrict__ v8t,
    const float* __restrict__ sq, const float* __restrict__ sk, const float* __restrict__ sv,
    const int32_t* __restrict__ idx, const float* __restrict__ alpha,
    const __bf16* __restrict__ t_g, const float* __restrict__ Z, const float* __restrict__ zb,
    float* __restrict__ O, int N, int nb, int topk, float c_log2,
    const int32_t* __restrict__ pairs = nullptr) {
  static_assert(D == 128, "the fp8 kernel is compiled for d = 128");
  constexpr int NS = D / 16, NC = D / 32, N8 = D / 64;
  constexpr int K8B = kBlock * D;  // bytes of a K8 (or V8^T) tile
  constexpr int kMaxWords = 64;    // union bitmap words: n_b <= 2048
  constexpr float QMAX = fmt_max<FMT>();
  // products over the head dim: N8 steps of 64-deep products of 32-byte operand chunks, in fp32
  auto dot64 = [](const i32x8* a, const i32x8* b) -> f32x16 {
    if constexpr (FMT == kFmtInt8) {
      i32x16 acc = i32x16{};
#pragma unroll
      for (int st = 0; st < N8; ++st) acc = mfma_i8x64(a[st], b[st], acc);
      return i2f16(acc);
    } else {
      f32x16 acc = f32x16{};
#pragma unroll
      for (int st = 0; st < N8; ++st) acc = mfma_f8(a[st], b[st], acc);
      return acc;
    }
  };
  // one 64-deep product (the PV step: 64 keys)
  auto dot1 = [](i32x8 a, i32x8 b) -> f32x16 {
    if constexpr (FMT == kFmtInt8)
      return i2f16(mfma_i8x64(a, b, i32x16{}));
    else
      return mfma_f8(a, b, f32x16{});
  };
  // K8 and V8^T tiles double-buffered, one LDS array each so that the compiler can tell the
  // buffers being filled by direct-to-LDS loads from the ones being read
  __shared__ __attribute__((aligned(16))) uint8_t kb0[K8B];
  __shared__ __attribute__((aligned(16))) uint8_t kb1[K8B];
  __shared__ __attribute__((aligned(16))) uint8_t vb0[K8B];
  __shared__ __attribute__((aligned(16))) uint8_t vb1[K8B];
  __shared__ uint32_t bm[2][kMaxWords];
  __shared__ int32_t ul[kMaxWords * 32];  // the union, ascending: (j << 2) | kept-by mask
  __shared__ int32_t ucount;
  __shared__ int32_t sl[2][kMaxWords * 32];  // the two kept lists (pass 1 reads them from here)
  __shared__ float zeta[2][D];
  __shared__ float tmx[2][2][2];  // [step parity][block][wavefront half]: partial P tile maxima
  __shared__ float qam[2][2];     // [block][wavefront half]: Q absmax (in-kernel quantisation)
  auto kbuf = [&](auto BUFC) -> uint8_t* { return decltype(BUFC)::value ? kb1 : kb0; };
  auto vbuf = [&](auto BUFC) -> uint8_t* { return decltype(BUFC)::value ? vb1 : vb0; };
  using B0 = std::integral_constant<int, 0>;
  using B1 = std::integral_constant<int, 1>;

  const int tid = threadIdx.x;
  const int lane = tid % kWave, g = lane / 32;
  const int w = __builtin_amdgcn_readfirstlane(tid / kWave);  // wavefront-uniform (scalar branches)
  const int item = xcd_remap(blockIdx.x, gridDim.x);
  const int npair = (nb + 1) / 2;
  const int bh = item / npair, pr = item % npair;
  // the two query blocks: 2p and 2p + 1, or (pairs) the ones matched by the overlap of their
  // kept sets; an odd n_b (or matching window) leaves one block alone, the absent second block
  // taking the id n_b (all its rows lie past N)
  int qa = 2 * pr, qbv = 2 * pr + 1;
  if (pairs) {
    qa = pairs[2 * ((size_t)bh * npair + pr)];
    qbv = pairs[2 * ((size_t)bh * npair + pr) + 1];
  }
  const bool has1 = pairs ? qbv >= 0 : qbv < nb;
  const int qb1 = has1 ? qbv : nb;
  auto qsel = [&](int b) { return b ? qb1 : qa; };
  const int blk = w / 2, half = w % 2;
  const bool present = blk == 0 || has1;  // the second block of a lone block's pair is absent
  const int qb = min(qsel(blk), nb - 1);
  const size_t hoff = (size_t)bh * N * D;
  const int nw = (nb + 31) / 32;

  // ---- the union of the two ascending index lists, with the kept-by bits ----
  if (tid < 2 * kMaxWords) bm[tid / kMaxWords][tid % kMaxWords] = 0u;
  __syncthreads();
  for (int t = tid; t < 2 * topk; t += kF8Threads) {
    const int b = t / topk;
    if (b == 0 || has1) {
      const int j = idx[((size_t)bh * nb + qsel(b)) * topk + t % topk];
      atomicOr(&bm[b][j / 32], 1u << (j % 32));
      sl[b][t % topk] = j;
    }
  }
  __syncthreads();
  if (w == 0) {
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

  // this wavefront's 32 rows (absent rows read a clamped one and are zeroed)
  const int m = 32 * half + lane % 32;
  const int row = qsel(blk) * kBlock + m;
  const bool row_ok = row < N;
  const bool rows_all_ok = __ballot(!row_ok) == 0;  // every row of this wavefront exists
  i32x8 qf[N8];  // e4m3 Q as the B operand: k-slot 32g + b of step s <-> channel 64s + 32g + b
  float sqi;
  if (q8) {  // codes and scales from the stand-alone quantiser
    const uint8_t* qr = q8 + hoff + (size_t)min(row, N - 1) * D + 32 * g;
#pragma unroll
    for (int st = 0; st < N8; ++st) {
      const i32x4* pq = reinterpret_cast<const i32x4*>(qr + 64 * st);
      qf[st] = row_ok ? join8(pq[0], pq[1]) : i32x8{};
    }
    sqi = sq[(size_t)bh * nb + qb];
  } else {
    // q8 null (grid-uniform): this workgroup quantises its own two query blocks, the only
    // workgroup that reads them, with the shared quantiser helpers (the same codes and scale):
    // each wavefront's absmax over its 32 rows meets its partner's in LDS
    i32x4 qv[N8][4];  // channels 64 st + 32 g + 8 i .. + 7 of this lane's row, bf16
    const __bf16* qr = Q + hoff + (size_t)min(row, N - 1) * D + 32 * g;
    float am = 0.f;
#pragma unroll
    for (int st = 0; st < N8; ++st) {
#pragma unroll
      for (int i = 0; i < 4; ++i) qv[st][i] = row_ok ? ld16(qr + 64 * st + 8 * i) : i32x4{0, 0, 0, 0};
      am = fmaxf(am, qz_local_amax(qv[st]));
    }
    am = wave_max(am);
    if (lane == 0) qam[blk][half] = am;
    __syncthreads();
    const float amax = fmaxf(qam[blk][0], qam[blk][1]);
    const float inv = qz_inv<FMT>(amax);
    sqi = qz_scale<FMT>(amax);
#pragma unroll
    for (int st = 0; st < N8; ++st) {
      uint2 c[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) c[i] = qz_row_codes<FMT>(qv[st][i], inv);
      qf[st] = i32x8{(int)c[0].x, (int)c[0].y, (int)c[1].x, (int)c[1].y,
                     (int)c[2].x, (int)c[2].y, (int)c[3].x, (int)c[3].y};
    }
  }

  // ---- pass 1: each row's exact maximum of S (log2 units) over its block's kept tiles (list
  // from LDS); K8 operands, the K scale and z_j from memory one tile ahead (rows past a short
  // block's end re-read its last row: those keys are masked); z_j of the kept blocks summed by
  // thread tid < D for block 0 and D .. 2D - 1 for block 1, i.e. each wavefront's own block ----
  const int32_t* sel = sl[blk];
  const int nsel = present ? topk : 0;
  auto k8_regs = [&](int j, i32x8 (&kr)[2][N8]) {
    const int nv = min(kBlock, N - j * kBlock);
    const uint8_t* src = k8 + hoff + (size_t)j * kBlock * D;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int st = 0; st < N8; ++st) {
        const i32x4* p = reinterpret_cast<const i32x4*>(src + (size_t)min(32 * kt + lane % 32, nv - 1) * D + 64 * st + 32 * g);
        kr[kt][st] = join8(p[0], p[1]);
      }
  };
  float mrow = -INFINITY, zacc = 0.f;
  {
    i32x8 kr[2][2][N8];
    // z_j and the K scale of the tile in kr[b], loaded with it (used right after a load, they
    // would make the compiler wait for every load in flight, the prefetch included)
    float zr[2], skr[2];
    auto step1 = [&](int t, auto BUFC) {
      constexpr int BUF = decltype(BUFC)::value;
      const int j = sel[t];
      zacc += zr[BUF];
      const float sc = sqi * skr[BUF] * c_log2;
      // the next tile's operands, unconditionally (the last step re-reads its own tile): a load
      // under a branch makes the compiler wait for every load in flight at the join
      const int jn = sel[min(t + 1, nsel - 1)];
      k8_regs(jn, kr[1 - BUF]);
      zr[1 - BUF] = zb[((size_t)bh * nb + jn) * D + tid % D];
      skr[1 - BUF] = sk[(size_t)bh * nb + jn];
      const int nv = min(kBlock, N - __builtin_amdgcn_readfirstlane(j) * kBlock);
      if (nv == kBlock) {  // a full tile: no key mask; sc > 0 scales the maximum once
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
          const f32x16 s = dot64(kr[BUF][kt], qf);
          float mx = s[0];
#pragma unroll
          for (int i = 1; i < 16; ++i) mx = fmaxf(mx, s[i]);
          mrow = fmaxf(mrow, mx * sc);
        }
      } else {
        const int lim = nv - 4 * g;
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
          const f32x16 s = dot64(kr[BUF][kt], qf);
#pragma unroll
          for (int i = 0; i < 16; ++i)
            if (32 * kt + 8 * (i / 4) + i % 4 < lim) mrow = fmaxf(mrow, s[i] * sc);
        }
      }
    };
    if (nsel > 0) {
      k8_regs(sel[0], kr[0]);
      zr[0] = zb[((size_t)bh * nb + sel[0]) * D + tid % D];
      skr[0] = sk[(size_t)bh * nb + sel[0]];
    }
    for (int t = 0; t < nsel; t += 2) {
      step1(t, B0{});
      if (t + 1 < nsel) step1(t + 1, B1{});
    }
  }
  mrow = xor32_max(mrow);

  // ---- pass 2 ----
  auto stage_k = [&](int t, uint8_t* dst) {
    const int j = ul[t] >> 2;
    const int nv = min(kBlock, N - j * kBlock);
    const uint8_t* src = k8 + hoff + (size_t)j * kBlock * D;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int r0 = 8 * (2 * w + u);  // 8 K8 rows of 128 B per wave load
      const int r = r0 + lane / 8;
      const int unit = (lane % 8) ^ ((r >> 1) & 7);
      load_lds16(src + (size_t)min(r, nv - 1) * D + unit * 16, dst + r0 * 128);
    }
  };
  auto stage_v = [&](int t, uint8_t* dst) {
    const int j = ul[t] >> 2;
    const uint8_t* src = v8t + ((size_t)bh * nb + j) * D * kBlock;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int c0 = 16 * (2 * w + u);  // 16 V8^T rows of 64 B per wave load
      const int c = c0 + lane / 4;
      const int vunit = (lane % 4) ^ ((c >> 2) & 3);
      load_lds16(src + (size_t)c * kBlock + vunit * 16, dst + c0 * 64);
    }
  };
  f32x16 os[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) os[c] = f32x16{};
  float lsum = 0.f;
  // S of the previous tile (keys past a short block and absent rows at -inf) and its score scale:
  // P is formed one step late, once the 64 x 64 tile's largest P^ is known
  f32x16 ss[2];
  float sc_prev = 0.f;
  bool prev_kept = false;
  int j_prev = 0;
  // log2 of the largest code (448 for e4m3, 127 for int8)
  constexpr float LOG2_QMAX = FMT == kFmtInt8 ? 6.98868468677216585f : 8.80735492205760410f;
  // P and PV of the previous tile from vbuf(VB), with its largest P^ from tmx[PB]: tmx holds
  // each half's max over rows of (row's tile maximum of S sc - the row's exact maximum), i.e. the
  // log2 of the tile's largest P^ = 2^(S sc - m).  The code's argument P^ QMAX / max(tile) is
  // then one exponential, 2^(S sc - m + log2 QMAX - e), and the tile's scale sP = 2^e / QMAX.
  auto pv_prev = [&](auto VBC, auto PBC) {
    constexpr int PB = decltype(PBC)::value;
    const float e = fmaxf(tmx[PB][blk][0], tmx[PB][blk][1]);
    if (e == -INFINITY) return;  // every P^ underflows: the tile adds 0 (workgroup-uniform per block)
    const float bias = LOG2_QMAX - e - mrow;
    const uint8_t* vs = vbuf(VBC);
    i32x8 va[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const int cr = 32 * c + lane % 32;
      va[c] = join8(*reinterpret_cast<const i32x4*>(vs + v8_off(cr, 32 * g)),
                    *reinterpret_cast<const i32x4*>(vs + v8_off(cr, 32 * g + 16)));
    }
    // P8 as the B operand: slot 16kt + i <-> key 32kt + 8(i/4) + 4g + i%4
    i32x8 pf;
    float ysum = 0.f;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int qd = 0; qd < 4; ++qd) {
        float y[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          y[u] = fast_exp2(fmaf(ss[kt][4 * qd + u], sc_prev, bias));
          ysum += y[u];
        }
        if constexpr (FMT == kFmtInt8)  // y in [0, 127]: codes 0 .. 127
          pf[4 * kt + qd] = (int)cvt4_u7(y[0], y[1], y[2], y[3], 1.f);
        else  // y >= 0; one rounding above 448 is clamped back to it
          pf[4 * kt + qd] = (int)cvt4_e4m3(fminf(y[0], kE4M3Max), fminf(y[1], kE4M3Max),
                                           fminf(y[2], kE4M3Max), fminf(y[3], kE4M3Max));
      }
    const float sp = fast_exp2(e - LOG2_QMAX);  // the tile's scale max / QMAX
    lsum = fmaf(ysum, sp, lsum);                // the unquantised P^ = y sP
    const float pv_scale = sp * sv[(size_t)bh * nb + j_prev];
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const f32x16 tmp = dot1(va[c], pf);
      os[c] += tmp * pv_scale;
    }
  };
  if (nu > 0) {
    stage_k(0, kb0);
    wait_vmem();
    __syncthreads();
  }
  // every path into the loop has waited for the operands loaded into registers above (else the
  // compiler waits for all memory traffic, the next tile's prefetch included, in every step)
  wait_vmem();
  // step t: K(t) in kbuf(B) (B = t & 1), V(t - 1) in vbuf(1 - B); stage K(t + 1) and V(t)
  auto step2 = [&](int t, auto BUFC) {
    constexpr int BUF = decltype(BUFC)::value;
    using OTHER = std::integral_constant<int, 1 - BUF>;
    if (t + 1 < nu) stage_k(t + 1, kbuf(OTHER{}));
    stage_v(t, vbuf(BUFC));
    if (prev_kept) pv_prev(OTHER{}, OTHER{});
    const int e = ul[t];
    const int j = e >> 2;
    const bool kept = (e >> blk) & 1;  // wavefront-uniform
    float emax = -INFINITY;
    if (kept) {
      const float sc = sqi * sk[(size_t)bh * nb + j] * c_log2;
      const int nv = min(kBlock, N - j * kBlock);
      const int lim = row_ok ? nv - 4 * g : 0;
      const bool full = rows_all_ok && nv == kBlock;  // wavefront-uniform: no key or row mask
      const uint8_t* ks = kbuf(BUFC);
      float amax = -INFINITY;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        i32x8 ka[N8];
#pragma unroll
        for (int st = 0; st < N8; ++st) {
          const int r = 32 * kt + lane % 32;
          const i32x4 a0 = *reinterpret_cast<const i32x4*>(ks + k8_off(r, 64 * st + 32 * g));
          const i32x4 a1 = *reinterpret_cast<const i32x4*>(ks + k8_off(r, 64 * st + 32 * g + 16));
          ka[st] = join8(a0, a1);
        }
        f32x16 s = dot64(ka, qf);
        if (!full) {
#pragma unroll
          for (int i = 0; i < 16; ++i)
            if (32 * kt + 8 * (i / 4) + i % 4 >= lim) s[i] = -INFINITY;
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) amax = fmaxf(amax, s[i]);
        ss[kt] = s;
      }
      // log2 of this row's largest P^ in the tile (sc > 0), then the max over the 32 rows
      emax = wave_max(amax * sc - mrow);
      sc_prev = sc;
    }
    if (lane == 0) tmx[BUF][blk][half] = emax;
    prev_kept = kept;
    j_prev = j;
    wait_vmem();
    __syncthreads();
  };
  for (int t = 0; t < nu; t += 2) {
    step2(t, B0{});
    if (t + 1 < nu) step2(t + 1, B1{});
  }
  // the last tile's PV: its V and both partial maxima are in since the last barrier
  if (prev_kept) {
    if ((nu - 1) & 1)
      pv_prev(B1{}, B1{});
    else
      pv_prev(B0{}, B0{});
  }

  // ---- epilogue: zeta, relu(Q) T_i with T_i^T rows read from memory, combine ----
  if (tid < 2 * D) zeta[blk][tid % D] = Z[(size_t)bh * D + tid % D] - zacc;
  bf16x8 qv[NS];
  {
    const __bf16* qr = Q + hoff + (size_t)min(row, N - 1) * D + 8 * g;
#pragma unroll
    for (int k = 0; k < NS; ++k) qv[k] = *reinterpret_cast<const bf16x8*>(qr + 16 * k);
  }
  __syncthreads();
  const float ltot = xor32_sum(lsum);
  const float inv_l = ltot > 0.f ? 1.f / ltot : 0.f;
  // num^T[c][m] = sum_c' T_i^T[c][c'] relu(Q)[m][c']: the A operand (rows c, k = c') is row c of
  // T_i^T, 16 bytes per lane and step, from memory (L2: both wavefronts of a block read it)
  const __bf16* tt = t_g + ((size_t)bh * nb + qb) * D * D;
  f32x16 num[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) num[c] = f32x16{};
  float den = 0.f;
#pragma unroll
  for (int k = 0; k < NS; ++k) {
    const bf16x8 pq = relu8(row_ok ? qv[k] : bf16x8{});
    bf16x8 ta[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c)
      ta[c] = *reinterpret_cast<const bf16x8*>(tt + (size_t)(32 * c + lane % 32) * D + 16 * k + 8 * g);
#pragma unroll
    for (int c = 0; c < NC; ++c) num[c] = mfma32(ta[c], pq, num[c]);
#pragma unroll
    for (int jj = 0; jj < 8; ++jj) den += bf2f(pq[jj]) * zeta[blk][16 * k + 8 * g + jj];
  }
  den = xor32_sum(den);
  const float inv_den = (topk < nb && den != 0.f) ? 1.f / den : 0.f;
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
      for (int e = 0; e < 4; ++e) v[e] = fmaf(num[c][4 * qd + e], wl, os[c][4 * qd + e] * ws);
      *reinterpret_cast<f32x4*>(orow + 32 * c + 8 * qd + 4 * g) = v;
    }
}

}  // namespace

hipError_t launch_quantize(const Dims& p, const void* X, uint8_t* codes, float* scales,
                           hipStream_t stream, int int8) {
  dim3 grid(p.nb, p.B * p.H);
  if (int8)
    quantize_kernel<128, false, kFmtInt8><<<grid, 256, 0, stream>>>((const __bf16*)X, p.N, p.nb, codes, scales);
  else
    quantize_kernel<128, false, kFmtE4M3><<<grid, 256, 0, stream>>>((const __bf16*)X, p.N, p.nb, codes, scales);
  return hipGetLastError();
}

hipError_t launch_quantize_v8t(const Dims& p, const void* X, uint8_t* codes, float* scales,
                               hipStream_t stream, int int8) {
  dim3 grid(p.nb, p.B * p.H);
  if (int8)
    quantize_kernel<128, true, kFmtInt8><<<grid, 256, 0, stream>>>((const __bf16*)X, p.N, p.nb, codes, scales);
  else
    quantize_kernel<128, true, kFmtE4M3><<<grid, 256, 0, stream>>>((const __bf16*)X, p.N, p.nb, codes, scales);
  return hipGetLastError();
}

hipError_t launch_sparse_fp8(const Dims& p, const void* Q, const void* K, const void* V,
                             const uint8_t* q8, const uint8_t* k8, const uint8_t* v8,
                             const float* sq, const float* sk, const float* sv,
                             const int32_t* idx, const float* alpha, const __bf16* ht_hi,
                             const __bf16* ht_lo, const float* Z, const float* zb, float* O,
                             hipStream_t stream) {
  const float c_log2 = 1.4426950408889634f / sqrtf((float)p.d);
  sparse_fp8_kernel<128><<<p.B * p.H * p.nb, kF8Threads, 0, stream>>>(
      (const __bf16*)Q, (const __bf16*)K, (const __bf16*)V, q8, k8, v8, sq, sk, sv, idx, alpha,
      ht_hi, ht_lo, Z, zb, O, p.N, p.nb, p.topk, c_log2);
  return hipGetLastError();
}

hipError_t launch_sparse_pair8(const Dims& p, const void* Q, const uint8_t* q8, const uint8_t* k8,
                               const uint8_t* v8, const float* sq, const float* sk,
                               const float* sv, const int32_t* idx, const float* alpha,
                               const __bf16* t_bf, const float* Z, const float* zb, float* O,
                               hipStream_t stream, int int8, const int32_t* pairs) {
  if (p.nb > 2048) return hipErrorInvalidValue;
  const float c_log2 = 1.4426950408889634f / sqrtf((float)p.d);
  const int grid = p.B * p.H * ((p.nb + 1) / 2);
  if (int8)
    pair8_kernel<128, kFmtInt8><<<grid, kF8Threads, 0, stream>>>(
        (const __bf16*)Q, q8, k8, v8, sq, sk, sv, idx, alpha, t_bf, Z, zb, O, p.N, p.nb, p.topk,
        c_log2, pairs);
  else
    pair8_kernel<128, kFmtE4M3><<<grid, kF8Threads, 0, stream>>>(
        (const __bf16*)Q, q8, k8, v8, sq, sk, sv, idx, alpha, t_bf, Z, zb, O, p.N, p.nb, p.topk,
        c_log2, pairs);
  return hipGetLastError();
}

}  // namespace sla
