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
//                     matches the P operand of the PV MFMA.
//   sparse_fp8_kernel one workgroup per query block, two wavefronts of 32 query rows.
//                     Pass 1 walks the kept blocks with S = Q8 K8^T (v_mfma ... f8f6f4,
//                     32x32x64) to get each row's exact maximum; pass 2 recomputes S, forms
//                     P = exp(S - max), the tile maximum across both wavefronts, P8, and
//                     O_s += (P8 V8) sP sV on fp8 MFMA, while the bf16 linear removal
//                     (relu(Q) relu(K_j)^T V_j) and the combine run as in the bf16 kernel.
#include "sla_device.hpp"
#include "sla_launch.hpp"
#include "sla_tiles.hpp"

namespace sla {

namespace {

constexpr float kE4M3Max = 448.f;

__device__ __forceinline__ f32x16 mfma_f8(i32x8 a, i32x8 b, f32x16 c) {
  // formats 0/0 = e4m3 for both operands; scale exponents 127 = 2^0
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

// e4m3 codes of 4 floats (round to nearest even; the caller keeps |x| <= 448)
__device__ __forceinline__ u32 cvt4_e4m3(float a, float b, float c, float d) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
  return (u32)w;
}
__device__ __forceinline__ float sat(float x) { return fminf(fmaxf(x, -kE4M3Max), kE4M3Max); }

// key position inside a transposed V8 row: lane group g of the PV MFMA reads bytes
// 32g .. 32g + 31, k-slot 16kt + 4q + e <-> key 32kt + 8q + 4g + e
__device__ __forceinline__ int v8_pos(int n) {
  const int kt = n / 32, q = (n % 32) / 8, g = (n % 8) / 4, e = n % 4;
  return 32 * g + 16 * kt + 4 * q + e;
}

template <int D, bool TRANSPOSED>
__global__ __launch_bounds__(256) void quantize_kernel(const __bf16* __restrict__ X, int N,
                                                       int nb, uint8_t* __restrict__ codes,
                                                       float* __restrict__ scales) {
  __shared__ float wmax[4];
  const int tid = threadIdx.x, lane = tid % kWave, w = tid / kWave;
  const int t = blockIdx.x, bh = blockIdx.y;
  const int row0 = t * kBlock;
  const int cnt = min(kBlock, N - row0);
  constexpr int CPR = D / 8;                  // 16-byte chunks per row
  constexpr int PER = kBlock * CPR / 256;     // chunks per thread
  const __bf16* Xb = X + ((size_t)bh * N + row0) * D;
  bf16x8 v[PER];
  float amax = 0.f;
#pragma unroll
  for (int u = 0; u < PER; ++u) {
    const int q = tid + u * 256, r = q / CPR, ch = q % CPR;
    v[u] = r < cnt ? *reinterpret_cast<const bf16x8*>(Xb + (size_t)r * D + ch * 8) : bf16x8{};
#pragma unroll
    for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(bf2f(v[u][e])));
  }
  amax = wave_max(amax);
  if (lane == 0) wmax[w] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]));
  const float inv = amax > 0.f ? kE4M3Max / amax : 0.f;
  if (tid == 0) scales[(size_t)bh * nb + t] = amax > 0.f ? amax / kE4M3Max : 1.f;
#pragma unroll
  for (int u = 0; u < PER; ++u) {
    const int q = tid + u * 256, r = q / CPR, ch = q % CPR;
    if (!TRANSPOSED && r >= cnt) continue;  // past N: no such row in the output
    float y[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) y[e] = sat(bf2f(v[u][e]) * inv);
    if constexpr (!TRANSPOSED) {
      const u32 lo = cvt4_e4m3(y[0], y[1], y[2], y[3]);
      const u32 hi = cvt4_e4m3(y[4], y[5], y[6], y[7]);
      uint8_t* dst = codes + ((size_t)bh * N + row0 + r) * D + ch * 8;
      *reinterpret_cast<uint2*>(dst) = make_uint2(lo, hi);
    } else {
      // [bh][t][c][pos(r)]; keys past N get code 0 (their P8 is 0 as well)
      uint8_t* dst = codes + ((size_t)bh * nb + t) * D * kBlock + v8_pos(r);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const u32 c = cvt4_e4m3(y[e], 0.f, 0.f, 0.f);
        dst[(size_t)(ch * 8 + e) * kBlock] = (uint8_t)(c & 0xff);
      }
    }
  }
}

constexpr int kF8Threads = 128;

template <int D>
__global__ __launch_bounds__(kF8Threads) void sparse_fp8_kernel(
    const __bf16* __restrict__ Q, const __bf16* __restrict__ K, const __bf16* __restrict__ V,
    const uint8_t* __restrict__ q8, const uint8_t* __restrict__ k8,
    const uint8_t* __restrict__ v8t, const float* __restrict__ sq,
    const float* __restrict__ sk, const float* __restrict__ sv,
    const int32_t* __restrict__ idx, const float* __restrict__ alpha,
    const __bf16* __restrict__ ht_hi, const __bf16* __restrict__ ht_lo,
    const float* __restrict__ Z, const float* __restrict__ zb, float* __restrict__ O, int N,
    int nb, int topk, float c_log2) {
  static_assert(D == 128, "the fp8 kernel is compiled for d = 128");
  constexpr int NS = D / 16, NC = D / 32, N8 = D / 64;
  constexpr int P8 = D + 16;  // LDS row pitch of the fp8 K tile in bytes
  __shared__ __attribute__((aligned(16))) __bf16 Ks[TileLayout<D>::ELEMS];
  __shared__ __attribute__((aligned(16))) __bf16 Vs[TileLayout<D>::ELEMS];
  __shared__ __attribute__((aligned(16))) uint8_t K8s[kBlock * P8];
  __shared__ __attribute__((aligned(16))) uint8_t V8s[D * (kBlock + 16)];
  __shared__ float zeta[D];
  __shared__ float tmax_x[2];

  const int tid = threadIdx.x;
  const int lane = tid % kWave, w = tid / kWave, g = lane / 32;
  const int item = xcd_remap(blockIdx.x, gridDim.x);
  const int bh = item / nb, qb = item % nb;
  const int m = 32 * w + lane % 32;
  const int row = qb * kBlock + m;
  const bool row_ok = row < N;
  const size_t hoff = (size_t)bh * N * D;
  const int32_t* sel = idx + ((size_t)bh * nb + qb) * topk;
  const float sqi = sq[(size_t)bh * nb + qb];

  // bf16 Q (linear branch) and e4m3 Q (sparse branch) as B operands
  bf16x8 pq[NS];
#pragma unroll
  for (int s = 0; s < NS; ++s)
    pq[s] = relu8(row_ok ? *reinterpret_cast<const bf16x8*>(Q + hoff + (size_t)row * D + 16 * s + 8 * g)
                         : bf16x8{});
  i32x8 qf[N8];
#pragma unroll
  for (int s = 0; s < N8; ++s) {
    if (row_ok) {
      const i32x4* p = reinterpret_cast<const i32x4*>(q8 + hoff + (size_t)row * D + 64 * s + 32 * g);
      const i32x4 a = p[0], b = p[1];
      qf[s] = i32x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
    } else {
      qf[s] = i32x8{};
    }
  }

  // load an fp8 K tile (row-major, pitch P8) into LDS: 64 rows x D bytes
  auto load_k8 = [&](int j) {
    const uint8_t* src = k8 + hoff + (size_t)j * kBlock * D;
    const int nv = min(kBlock, N - j * kBlock);
    for (int q = tid; q < kBlock * D / 16; q += kF8Threads) {
      const int r = q / (D / 16), ch = q % (D / 16);
      const i32x4 v = r < nv ? *reinterpret_cast<const i32x4*>(src + (size_t)r * D + ch * 16)
                             : i32x4{0, 0, 0, 0};
      *reinterpret_cast<i32x4*>(K8s + r * P8 + ch * 16) = v;
    }
  };
  auto s_tile = [&](f32x16* s) {
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      s[kt] = f32x16{};
#pragma unroll
      for (int st = 0; st < N8; ++st) {
        const i32x4* p = reinterpret_cast<const i32x4*>(K8s + (32 * kt + lane % 32) * P8 + 64 * st + 32 * g);
        const i32x4 a = p[0], b = p[1];
        s[kt] = mfma_f8(i32x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]}, qf[st], s[kt]);
      }
    }
  };

  // ---- pass 1: exact row maximum of S (log2 units) over all kept keys ----
  float mrow = -INFINITY;
  for (int t = 0; t < topk; ++t) {
    const int j = sel[t];
    const int nv = min(kBlock, N - j * kBlock);
    __syncthreads();
    load_k8(j);
    __syncthreads();
    f32x16 s[2];
    s_tile(s);
    const float sc = sqi * sk[(size_t)bh * nb + j] * c_log2;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int i = 0; i < 16; ++i)
        if (32 * kt + 8 * (i / 4) + 4 * g + i % 4 < nv) mrow = fmaxf(mrow, s[kt][i] * sc);
  }
  mrow = fmaxf(mrow, __shfl_xor(mrow, 32));

  // ---- pass 2 ----
  f32x16 os[NC], ol[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    os[c] = f32x16{};
    ol[c] = f32x16{};
  }
  float lsum = 0.f, zacc = 0.f;
  TileLoader<__bf16, D, kF8Threads> lk, lv;
  for (int t = 0; t < topk; ++t) {
    const int j = sel[t];
    const int nv = min(kBlock, N - j * kBlock);
    lk.load(K + hoff + (size_t)j * kBlock * D, nv, tid);
    lv.load(V + hoff + (size_t)j * kBlock * D, nv, tid);
    __syncthreads();
    load_k8(j);
    {  // transposed V8 block [D][64] -> LDS rows padded to 80 bytes
      const uint8_t* src = v8t + ((size_t)bh * nb + j) * D * kBlock;
      for (int q = tid; q < D * kBlock / 16; q += kF8Threads) {
        const int c = q / (kBlock / 16), ch = q % (kBlock / 16);
        *reinterpret_cast<i32x4*>(V8s + c * (kBlock + 16) + ch * 16) =
            *reinterpret_cast<const i32x4*>(src + (size_t)c * kBlock + ch * 16);
      }
    }
    lk.store(Ks, tid);
    lv.store(Vs, tid);
    if (tid < D) zacc += zb[((size_t)bh * nb + j) * D + tid];
    __syncthreads();

    f32x16 s[2];
    s_tile(s);
    const float sc = sqi * sk[(size_t)bh * nb + j] * c_log2;
    float p[2][16];
    float pmax = 0.f;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const bool ok = row_ok && 32 * kt + 8 * (i / 4) + 4 * g + i % 4 < nv;
        p[kt][i] = ok ? fast_exp2(fmaf(s[kt][i], sc, -mrow)) : 0.f;
        lsum += p[kt][i];
        pmax = fmaxf(pmax, p[kt][i]);
      }
    pmax = wave_max(pmax);
    if (lane == 0) tmax_x[w] = pmax;
    // linear removal on the bf16 tiles (independent of the tile maximum)
    f32x16 l[2];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      l[kt] = f32x16{};
#pragma unroll
      for (int st = 0; st < NS; ++st) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(Ks + TileLayout<D>::off(32 * kt + lane % 32, 16 * st + 8 * g));
        l[kt] = mfma32(relu8(a), pq[st], l[kt]);
      }
    }
#pragma unroll
    for (int c = 0; c < NC; ++c)
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        bf16x8 lb;
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) lb[jj] = f2bf(-l[u / 2][8 * (u % 2) + jj]);
        ol[c] = mfma32(tr_operand<D, 4, 8>(Vs, 16 * u, 32 * c, lane), lb, ol[c]);
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
      const i32x4* pa = reinterpret_cast<const i32x4*>(V8s + (32 * c + lane % 32) * (kBlock + 16) + 32 * g);
      const i32x4 a = pa[0], b = pa[1];
      const f32x16 tmp = mfma_f8(i32x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]}, pf, f32x16{});
      os[c] += tmp * pv_scale;
    }
  }

  // ---- epilogue (as in the bf16 kernel) ----
  const float ltot = lsum + __shfl_xor(lsum, 32);
  const float inv_l = topk > 0 ? 1.f / ltot : 0.f;
  __syncthreads();
  if (tid < D) zeta[tid] = Z[(size_t)bh * D + tid] - zacc;
  __syncthreads();
  const __bf16* hh = ht_hi + (size_t)bh * D * D;
  const __bf16* hl = ht_lo + (size_t)bh * D * D;
#pragma unroll
  for (int c = 0; c < NC; ++c)
#pragma unroll
    for (int st = 0; st < NS; ++st) {
      const size_t off = (size_t)(32 * c + lane % 32) * D + 16 * st + 8 * g;
      ol[c] = mfma32(*reinterpret_cast<const bf16x8*>(hl + off), pq[st], ol[c]);
      ol[c] = mfma32(*reinterpret_cast<const bf16x8*>(hh + off), pq[st], ol[c]);
    }
  float den = 0.f;
#pragma unroll
  for (int st = 0; st < NS; ++st)
#pragma unroll
    for (int jj = 0; jj < 8; ++jj) den += bf2f(pq[st][jj]) * zeta[16 * st + 8 * g + jj];
  den += __shfl_xor(den, 32);
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
      for (int e = 0; e < 4; ++e) v[e] = fmaf(ol[c][4 * qd + e], wl, os[c][4 * qd + e] * ws);
      *reinterpret_cast<f32x4*>(orow + 32 * c + 8 * qd + 4 * g) = v;
    }
}

}  // namespace

hipError_t launch_quantize(const Dims& p, const void* X, uint8_t* codes, float* scales,
                           hipStream_t stream) {
  dim3 grid(p.nb, p.B * p.H);
  quantize_kernel<128, false><<<grid, 256, 0, stream>>>((const __bf16*)X, p.N, p.nb, codes, scales);
  return hipGetLastError();
}

hipError_t launch_quantize_v8t(const Dims& p, const void* X, uint8_t* codes, float* scales,
                               hipStream_t stream) {
  dim3 grid(p.nb, p.B * p.H);
  quantize_kernel<128, true><<<grid, 256, 0, stream>>>((const __bf16*)X, p.N, p.nb, codes, scales);
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

}  // namespace sla
