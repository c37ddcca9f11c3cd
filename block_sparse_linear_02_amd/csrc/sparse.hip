// sparse.hip - block-sparse softmax branch with the fused linear-branch removal and the alpha
// combine, on gfx950.
//
// Sources: SLA2 Italian summary sections 1 and 2.A and Arabic summary sections 1 and 2.alef
// (sparse branch renormalised over the kept blocks; O = alpha O_s + (1 - alpha) O_l); SALAD
// section 2 (ReLU feature map of the linear branch).
//
// One workgroup = one query block (64 rows) of one (batch, head); two wavefronts of 32 query
// rows each.  For every kept key block j (the router's ascending list):
//   * K_j and V_j arrive in LDS as row-major bf16 tiles (the next tile's global loads are in
//     flight while the current one is used);
//   * S^T = K_j Q^T by v_mfma_f32_32x32x16_bf16 with Q held in registers (B operand), so each
//     lane owns one query row: row max / rescale / sum stay inside a lane (plus one exchange
//     with lane^32);
//   * online softmax in the log2 domain, P rounded to bf16;
//   * O_s^T += V_j^T P^T, the V operand read transposed from LDS (ds_read_b64_tr_b16);
//   * fused linear removal: L^T = relu(K_j) relu(Q)^T on the same K registers and
//     O_l^T -= V_j^T L^T on the same V registers, i.e. sum over kept blocks of
//     relu(Q) h_j = (relu(Q) relu(K_j)^T) V_j without reading the d x d state h_j.
// Epilogue: O_l numerator += relu(Q) H (H^T split bf16 hi + lo, MFMA), denominator
// relu(q) . (Z - sum_kept z_j), O = alpha O_s / l + (1 - alpha) num / den (0 if nothing is
// unselected or den == 0), fp32 stores; rows past N are not stored.
#include "sla_device.hpp"
#include "sla_launch.hpp"
#include "sla_tiles.hpp"

namespace sla {

namespace {

constexpr int kSparseThreads = 128;

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

template <class T, int D, bool FUSED>
__global__ __launch_bounds__(kSparseThreads) void sparse_kernel(
    const T* __restrict__ Q, const T* __restrict__ K, const T* __restrict__ V,
    const int32_t* __restrict__ idx, const float* __restrict__ alpha,
    const __bf16* __restrict__ ht_hi, const __bf16* __restrict__ ht_lo,
    const float* __restrict__ Z, const float* __restrict__ zb, float* __restrict__ O, int N,
    int nb, int topk, float c_log2) {
  constexpr int NS = D / 16;  // MFMA k-steps over the head dim
  constexpr int NC = D / 32;  // 32-channel output tiles
  __shared__ __attribute__((aligned(16))) __bf16 Ks[kBlock * (D + kPad)];
  __shared__ __attribute__((aligned(16))) __bf16 Vs[kBlock * (D + kPad)];
  __shared__ float zeta[D];

  const int tid = threadIdx.x;
  const int lane = tid % kWave, w = tid / kWave, g = lane / 32;
  const int item = xcd_remap(blockIdx.x, gridDim.x);
  const int bh = item / nb, qb = item % nb;
  const int m = 32 * w + lane % 32;  // this lane's query row inside the block
  const int row = qb * kBlock + m;
  const bool row_ok = row < N;
  const size_t hoff = (size_t)bh * N * D;
  const int32_t* sel = idx + ((size_t)bh * nb + qb) * topk;

  // Q rows as the B operand of S^T = K Q^T: k-slot 8g + jj of step s <-> channel 16s + 8g + jj
  bf16x8 q[NS], pq[NS];
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    q[s] = row_ok ? load_row8<T>(Q + hoff + (size_t)row * D + 16 * s + 8 * g) : bf16x8{};
    pq[s] = relu8(q[s]);
  }

  f32x16 os[NC], ol[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    os[c] = f32x16{};
    ol[c] = f32x16{};
  }
  float mrun = -INFINITY, lsum = 0.f;
  float zacc = 0.f;  // thread tid < D: sum of z_j over the kept blocks, channel tid

  TileLoader<T, D, kSparseThreads> lk, lv;
  if (topk > 0) {
    const int j = sel[0];
    const int nv = min(kBlock, N - j * kBlock);
    lk.load(K + hoff + (size_t)j * kBlock * D, nv, tid);
    lv.load(V + hoff + (size_t)j * kBlock * D, nv, tid);
  }

  for (int t = 0; t < topk; ++t) {
    const int j = sel[t];
    const int nv = min(kBlock, N - j * kBlock);
    __syncthreads();  // the previous tile is consumed
    lk.store(Ks, tid);
    lv.store(Vs, tid);
    __syncthreads();
    if (t + 1 < topk) {
      const int jn = sel[t + 1];
      const int nvn = min(kBlock, N - jn * kBlock);
      lk.load(K + hoff + (size_t)jn * kBlock * D, nvn, tid);
      lv.load(V + hoff + (size_t)jn * kBlock * D, nvn, tid);
    }
    if (FUSED && tid < D) zacc += zb[((size_t)bh * nb + j) * D + tid];

    // S^T (and L^T) for the two 32-key halves of the tile
    f32x16 s[2], l[2];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      s[kt] = f32x16{};
      l[kt] = f32x16{};
#pragma unroll
      for (int st = 0; st < NS; ++st) {
        const bf16x8 a =
            *reinterpret_cast<const bf16x8*>(Ks + (32 * kt + lane % 32) * (D + kPad) + 16 * st + 8 * g);
        s[kt] = mfma32(a, q[st], s[kt]);
        if constexpr (FUSED) l[kt] = mfma32(relu8(a), pq[st], l[kt]);
      }
    }
    // key of accumulator register i in half kt: 32kt + 8(i/4) + 4g + i%4
    if (nv < kBlock) {
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (32 * kt + 8 * (i / 4) + 4 * g + i % 4 >= nv) s[kt][i] = -INFINITY;
    }
    // online softmax (log2 domain)
    float mx = -INFINITY;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[kt][i]);
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float mnew = fmaxf(mrun, mx * c_log2);
    const float corr = fast_exp2(mrun - mnew);
    mrun = mnew;
    float psum = 0.f;
    bf16x8 pb[4], lb[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) {
        const float p = fast_exp2(fmaf(s[u / 2][8 * (u % 2) + jj], c_log2, -mnew));
        psum += p;
        pb[u][jj] = f2bf(p);
        if constexpr (FUSED) lb[u][jj] = f2bf(-l[u / 2][8 * (u % 2) + jj]);
      }
    }
    lsum = lsum * corr + psum;
    if (__ballot(corr != 1.f)) {
#pragma unroll
      for (int c = 0; c < NC; ++c) os[c] *= corr;
    }
    // O^T += V^T P^T (and the linear removal) ; MFMA u covers keys 16u .. 16u + 15
#pragma unroll
    for (int c = 0; c < NC; ++c)
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const bf16x8 av = tr_operand<D, 4, 8>(Vs, 16 * u, 32 * c, lane);
        os[c] = mfma32(av, pb[u], os[c]);
        if constexpr (FUSED) ol[c] = mfma32(av, lb[u], ol[c]);
      }
  }

  // ---- epilogue ----
  const float ltot = lsum + __shfl_xor(lsum, 32);
  const float inv_l = topk > 0 ? 1.f / ltot : 0.f;
  float inv_den = 0.f;
  if constexpr (FUSED) {
    if (tid < D) zeta[tid] = Z[(size_t)bh * D + tid] - zacc;
    __syncthreads();
    // numerator += relu(Q) H : A = H^T rows (V channel c), k-slots = K channel c'
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
        v[e] = FUSED ? fmaf(ol[c][4 * qd + e], wl, x) : x;
      }
      *reinterpret_cast<f32x4*>(orow + 32 * c + 8 * qd + 4 * g) = v;
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
