// linear_apply.hip - the literal form of the ReLU linear branch on gfx950: per query block i,
//   A_i = H - sum_{j kept} h_j,   zeta_i = Z - sum_{j kept} z_j,
//   O_l(q) = relu(q) A_i / (relu(q) . zeta_i)
// (SALAD section 2 for relu; SLA2 Italian summary section 1: the linear branch covers the
// blocks the sparse branch does not keep), added to O as (1 - alpha) O_l.  O already holds
// alpha O_s from the sparse kernel.
//
// One workgroup per query block: the kept blocks' d x d states are summed in fp32 with
// coalesced reads (k * (d^2 + d) * 4 bytes per query block - the cost this form pays), A_i and
// relu(Q_i) are staged in LDS, and each thread forms a row x (d/4 channels) slice of the
// product on the fp32 VALU.
#include "sla_device.hpp"
#include "sla_launch.hpp"
#include "sla_tiles.hpp"

namespace sla {

namespace {

constexpr int kLitThreads = 256;

template <class T, int D>
__global__ __launch_bounds__(kLitThreads) void linear_literal_kernel(
    const T* __restrict__ Q, const int32_t* __restrict__ idx, const float* __restrict__ alpha,
    const float* __restrict__ h_full, const float* __restrict__ Z, const float* __restrict__ hj,
    const float* __restrict__ zb, float* __restrict__ O, int N, int nb, int topk) {
  extern __shared__ float sm[];
  float* A = sm;                          // [D][D]  (K channel c', V channel c)
  float* qs = A + D * D;                  // [64][D + 1] relu(Q)
  float* zeta = qs + kBlock * (D + 1);    // [D]
  const int tid = threadIdx.x;
  const int item = xcd_remap(blockIdx.x, gridDim.x);
  const int bh = item / nb, qb = item % nb;
  const int32_t* sel = idx + ((size_t)bh * nb + qb) * topk;
  const float* hb = hj + (size_t)bh * nb * D * D;

  for (int e = tid; e < D * D; e += kLitThreads) {
    float s = 0.f;
    for (int t = 0; t < topk; ++t) s += hb[(size_t)sel[t] * D * D + e];
    A[e] = h_full[(size_t)bh * D * D + e] - s;
  }
  if (tid < D) {
    float s = 0.f;
    for (int t = 0; t < topk; ++t) s += zb[((size_t)bh * nb + sel[t]) * D + tid];
    zeta[tid] = Z[(size_t)bh * D + tid] - s;
  }
  const size_t hoff = (size_t)bh * N * D;
  for (int e = tid; e < kBlock * D; e += kLitThreads) {
    const int r = e / D, c = e % D;
    const int row = qb * kBlock + r;
    qs[r * (D + 1) + c] = row < N ? fmaxf((float)Q[hoff + (size_t)row * D + c], 0.f) : 0.f;
  }
  __syncthreads();

  const int r = tid / 4, cg = tid % 4;
  const int row = qb * kBlock + r;
  float acc[D / 4];
#pragma unroll
  for (int k = 0; k < D / 4; ++k) acc[k] = 0.f;
  float den = 0.f;
  for (int cp = 0; cp < D; ++cp) {
    const float qv = qs[r * (D + 1) + cp];
    den += qv * zeta[cp];
#pragma unroll
    for (int k = 0; k < D / 4; ++k) acc[k] += qv * A[cp * D + cg + 4 * k];
  }
  if (row >= N || topk >= nb || den == 0.f) return;
  const float wl = (1.f - alpha[(size_t)bh * N + row]) / den;
  float* orow = O + hoff + (size_t)row * D;
#pragma unroll
  for (int k = 0; k < D / 4; ++k) orow[cg + 4 * k] += acc[k] * wl;
}

template <class T, int D>
hipError_t launch_lit_t(const Dims& p, const void* Q, const int32_t* idx, const float* alpha,
                        const float* h_full, const float* Z, const float* hj, const float* zb,
                        float* O, hipStream_t stream) {
  const size_t lds = ((size_t)D * D + (size_t)kBlock * (D + 1) + D) * sizeof(float);
  hipError_t e = hipFuncSetAttribute((const void*)linear_literal_kernel<T, D>,
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  linear_literal_kernel<T, D><<<p.B * p.H * p.nb, kLitThreads, lds, stream>>>(
      (const T*)Q, idx, alpha, h_full, Z, hj, zb, O, p.N, p.nb, p.topk);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_linear_literal(const Dims& p, const void* Q, const int32_t* idx,
                                 const float* alpha, const float* h_full, const float* Z,
                                 const float* hj, const float* zb, float* O,
                                 hipStream_t stream) {
  if (p.dtype == kBF16 && p.d == 128) return launch_lit_t<__bf16, 128>(p, Q, idx, alpha, h_full, Z, hj, zb, O, stream);
  if (p.dtype == kBF16 && p.d == 64) return launch_lit_t<__bf16, 64>(p, Q, idx, alpha, h_full, Z, hj, zb, O, stream);
  if (p.dtype == kF32 && p.d == 128) return launch_lit_t<float, 128>(p, Q, idx, alpha, h_full, Z, hj, zb, O, stream);
  return launch_lit_t<float, 64>(p, Q, idx, alpha, h_full, Z, hj, zb, O, stream);
}

}  // namespace sla
