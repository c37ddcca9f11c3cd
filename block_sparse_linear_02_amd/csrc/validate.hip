// validate.hip - debug check of kept-block index lists on gfx950.
//
// Source: SLA2 Italian summary section 2.B and Arabic summary section 2.ba (HardTop-k keeps
// topk key blocks per query block; every kernel that reads idx takes each row as an ascending
// list of distinct key blocks in [0, n_b)).
//
//   validate_idx_kernel  one workgroup of 1024 threads walks every row (B H n_b rows of topk
//                        entries) and counts the rows with an entry outside [0, n_b) or not
//                        strictly above the entry before it; the count goes to *bad (written
//                        once, by thread 0, so the word needs no clearing).  A debug path: the
//                        caller synchronises and reads the count before anything else runs.
#include "sla_device.hpp"
#include "sla_launch.hpp"

namespace sla {

namespace {

constexpr int kValidateThreads = 1024;

__global__ __launch_bounds__(kValidateThreads) void validate_idx_kernel(const int32_t* __restrict__ idx,
                                                                       long long rows, int topk, int nb,
                                                                       int* __restrict__ bad) {
  __shared__ int part[kValidateThreads / kWave];
  int cnt = 0;
  for (long long r = threadIdx.x; r < rows; r += kValidateThreads) {
    const int32_t* row = idx + r * topk;
    int prev = -1;
    bool ok = true;
    for (int t = 0; t < topk; ++t) {
      const int j = row[t];
      ok = ok && j > prev && j < nb;  // j > prev >= -1 also rules out negative entries
      prev = j;
    }
    cnt += ok ? 0 : 1;
  }
#pragma unroll
  for (int o = kWave / 2; o > 0; o >>= 1) cnt += __shfl_xor(cnt, o);
  if (threadIdx.x % kWave == 0) part[threadIdx.x / kWave] = cnt;
  __syncthreads();
  if (threadIdx.x == 0) {
    int s = 0;
    for (int w = 0; w < kValidateThreads / kWave; ++w) s += part[w];
    *bad = s;
  }
}

}  // namespace

hipError_t launch_validate_idx(const Dims& p, const int32_t* idx, int* bad, hipStream_t stream) {
  const long long rows = (long long)p.B * p.H * p.nb;
  validate_idx_kernel<<<1, kValidateThreads, 0, stream>>>(idx, rows, p.topk, p.nb, bad);
  return hipGetLastError();
}

}  // namespace sla
