// branch_drop.hip - per-head branch flags for alpha-driven branch dropping on gfx950.
//
// Source: "SALAD: Achieve High-Sparsity Attention via Efficient Linear Attention Tuning for Video
// Diffusion Transformer", section 2, Post-Tuning Branch Dropping (a linear branch whose scale is
// very low is removed at inference); in SLA2 (Italian summary section 2.A) the linear branch of
// token t is weighted by 1 - alpha_t and the sparse branch by alpha_t.
//
//   branch_flags_kernel  one workgroup per (batch, head): min and max of alpha over the N tokens
//                        (float4 loads, wave and LDS reductions), then the head's flags:
//                        kDropLinear when max(1 - alpha) <= tau, kDropSparse when
//                        max(alpha) <= tau (0 <= tau < 0.5, so never both).  The state, mask
//                        GEMM and attention kernels read the flags and skip the dropped
//                        branch's work for that head; nothing waits on the host.
#include "sla_device.hpp"
#include "sla_launch.hpp"

namespace sla {

namespace {

constexpr int kFlagThreads = 256;

__global__ __launch_bounds__(kFlagThreads) void branch_flags_kernel(const float* __restrict__ alpha,
                                                                    int N, float tau,
                                                                    uint32_t* __restrict__ flags) {
  __shared__ float red[2][kFlagThreads / kWave];
  const int bh = blockIdx.x;
  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  const float* a = alpha + (size_t)bh * N;
  float mn = INFINITY, mx = -INFINITY;
  // the head's row is 16-byte aligned only when N % 4 == 0: vector loads then, scalar otherwise
  if ((N & 3) == 0) {
    for (int t = 4 * tid; t < N; t += 4 * kFlagThreads) {
      const f32x4 v = *reinterpret_cast<const f32x4*>(a + t);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        mn = fminf(mn, v[e]);
        mx = fmaxf(mx, v[e]);
      }
    }
  } else {
    for (int t = tid; t < N; t += kFlagThreads) {
      mn = fminf(mn, a[t]);
      mx = fmaxf(mx, a[t]);
    }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    mn = fminf(mn, __shfl_xor(mn, o));
    mx = fmaxf(mx, __shfl_xor(mx, o));
  }
  if (lane == 0) {
    red[0][wave] = mn;
    red[1][wave] = mx;
  }
  __syncthreads();
  if (tid == 0) {
#pragma unroll
    for (int w = 1; w < kFlagThreads / kWave; ++w) {
      mn = fminf(mn, red[0][w]);
      mx = fmaxf(mx, red[1][w]);
    }
    // 1 - min(alpha) is exact wherever it can reach tau < 0.5 (Sterbenz)
    uint32_t f = 0;
    if (1.f - mn <= tau) f |= kDropLinear;
    if (mx <= tau) f |= kDropSparse;
    flags[bh] = f;
  }
}

}  // namespace

hipError_t launch_branch_flags(const Dims& p, const float* alpha, float tau, uint32_t* flags,
                               hipStream_t stream) {
  branch_flags_kernel<<<p.B * p.H, kFlagThreads, 0, stream>>>(alpha, p.N, tau, flags);
  return hipGetLastError();
}

}  // namespace sla
