// svoo.hip - SVOO online bidirectional co-clustering of queries and keys on gfx950, and the row
// permutations around the attention path.
//
// SVOO (Italian summary, section 2.B): queries and keys are partitioned jointly.  Keys go to
// the cluster whose current query centroid has the largest inner product with them, then the
// queries go to the cluster whose updated key centroid has; the alternation repeats.  C = n_b
// clusters, started from the block means of Q and K (the router's pooling, no projection).
//
//   assign_kernel    256 tokens per workgroup (64 per wavefront, the B operand of the MFMA,
//                    loaded once into registers); the centroids stream through LDS in chunks
//                    of 64 (hi and lo bf16 halves, double-buffered): affinity = x . hi + x . lo
//                    on bf16 MFMA with fp32 accumulation (about fp32 accuracy: x is exactly
//                    bf16, the centroid is hi + lo + O(2^-17 |c|)), running argmax per token
//                    (the lower index among equal affinities).
//   hist_kernel      per 512-token segment, the count of each cluster (LDS atomics).
//   scan_kernel      per head: cluster starts (exclusive scan of the totals) and, per segment,
//                    the first position of its tokens in each cluster.
//   order_kernel     one wavefront per segment, tokens in their original order 64 at a time:
//                    lanes with the same cluster take consecutive positions (ballot of the
//                    lanes sharing the first pending lane's cluster), so the permutation is
//                    the stable sort of the tokens by cluster.
//   centroid_kernel  one workgroup per (cluster, head): the mean of its members, summed in fp64
//                    in the sorted order (deterministic), rounded to fp32 and split hi + lo; an
//                    empty cluster keeps its previous centroid.
//   permute_kernel   rows gathered (y[p] = x[perm[p]]) or scattered (y[perm[p]] = x[p]).
// bf16 Q and K with d = 128.
#include "sla_device.hpp"
#include "sla_launch.hpp"
#include "sla_tiles.hpp"

namespace sla {

namespace {

constexpr int kSvD = 128;
constexpr int kAssignThreads = 256;
constexpr int kAssignTokens = 256;  // 64 per wavefront
constexpr int kSegTokens = 512;     // tokens per counting-sort segment
constexpr int kMaxClusters = 2048;
constexpr int kScanThreads = 1024;  // two clusters per thread

__global__ __launch_bounds__(kAssignThreads, 2) void assign_kernel(
    const __bf16* __restrict__ X, const __bf16* __restrict__ c_hi,
    const __bf16* __restrict__ c_lo, int N, int C, int32_t* __restrict__ assign) {
  constexpr int D = kSvD, NS = D / 16;
  constexpr int TILE = TileLayout<D>::ELEMS;
  __shared__ __attribute__((aligned(16))) __bf16 lds[2][2 * TILE];  // [buffer][hi tile | lo tile]
  const int tid = threadIdx.x, lane = tid % kWave, g = lane / 32;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int bh = blockIdx.y;
  const __bf16* ch = c_hi + (size_t)bh * C * D;
  const __bf16* cl = c_lo + (size_t)bh * C * D;
  const int nchunk = (C + kBlock - 1) / kBlock;

  auto stage = [&](int t, int buf) {
    const int valid = min(kBlock, C - kBlock * t);
    const size_t off = (size_t)kBlock * t * D;
    if (valid == kBlock) {
      load_tile_direct<kAssignThreads>(ch + off, lds[buf], tid);
      load_tile_direct<kAssignThreads>(cl + off, lds[buf] + TILE, tid);
    } else {  // rows past C re-read the last centroid; the argmax skips them
      load_tile_direct_clamped<kAssignThreads>(ch + off, lds[buf], tid, valid);
      load_tile_direct_clamped<kAssignThreads>(cl + off, lds[buf] + TILE, tid, valid);
    }
  };
  stage(0, 0);

  // this wavefront's 64 tokens as two B operands (k-slot 8 g + e of step s <-> channel
  // 16 s + 8 g + e); tokens past N are zero and store nothing
  const int tok0 = blockIdx.x * kAssignTokens + wave * 64;
  bf16x8 xr[2][NS];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int tok = tok0 + 32 * u + lane % 32;
    const __bf16* row = X + ((size_t)bh * N + min(tok, N - 1)) * D + 8 * g;
#pragma unroll
    for (int s = 0; s < NS; ++s)
      xr[u][s] = tok < N ? *reinterpret_cast<const bf16x8*>(row + 16 * s) : bf16x8{};
  }
  float best[2] = {-INFINITY, -INFINITY};
  int bidx[2] = {0, 0};
  const int ap = row_part(lane);
  wait_vmem();
  __syncthreads();

  for (int t = 0; t < nchunk; ++t) {
    const int buf = t & 1;
    if (t + 1 < nchunk) stage(t + 1, buf ^ 1);
    const __bf16* th = lds[buf];
    const __bf16* tl = th + TILE;
    // acc[h][u]: rows = centroids 64 t + 32 h + (8 (i / 4) + 4 g + i % 4), column = token
    f32x16 acc[2][2];
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int u = 0; u < 2; ++u) acc[h][u] = f32x16{};
#pragma unroll
    for (int s = 0; s < NS; ++s)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const bf16x8 ah = lds_row16(th, 32 * h * 256 + (ap ^ (32 * s)));
        const bf16x8 al = lds_row16(tl, 32 * h * 256 + (ap ^ (32 * s)));
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          acc[h][u] = mfma32(ah, xr[u][s], acc[h][u]);
          acc[h][u] = mfma32(al, xr[u][s], acc[h][u]);
        }
      }
    // ascending centroid index within the lane, so a strict > keeps the lowest among equals
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int c = kBlock * t + 32 * h + 8 * (i / 4) + 4 * g + i % 4;
#pragma unroll
        for (int u = 0; u < 2; ++u)
          if (c < C && acc[h][u][i] > best[u]) {
            best[u] = acc[h][u][i];
            bidx[u] = c;
          }
      }
    wait_vmem();
    __syncthreads();
  }
  // lanes l and l + 32 hold the same token over interleaved centroid rows
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const float ov = __shfl_xor(best[u], 32);
    const int oi = __shfl_xor(bidx[u], 32);
    if (ov > best[u] || (ov == best[u] && oi < bidx[u])) {
      best[u] = ov;
      bidx[u] = oi;
    }
    const int tok = tok0 + 32 * u + lane % 32;
    if (g == 0 && tok < N) assign[(size_t)bh * N + tok] = bidx[u];
  }
}

__global__ __launch_bounds__(256) void hist_kernel(const int32_t* __restrict__ assign, int N,
                                                   int C, int S, int32_t* __restrict__ hist) {
  __shared__ int h[kMaxClusters];
  const int s = blockIdx.x, bh = blockIdx.y, tid = threadIdx.x;
  for (int c = tid; c < C; c += 256) h[c] = 0;
  __syncthreads();
  const int t1 = min(N, (s + 1) * kSegTokens);
  for (int t = s * kSegTokens + tid; t < t1; t += 256) atomicAdd(&h[assign[(size_t)bh * N + t]], 1);
  __syncthreads();
  for (int c = tid; c < C; c += 256) hist[((size_t)bh * S + s) * C + c] = h[c];
}

// hist [BH][S][C] counts in, first positions out; start [BH][C + 1].
__global__ __launch_bounds__(kScanThreads) void scan_kernel(int32_t* __restrict__ hist, int N,
                                                            int C, int S,
                                                            int32_t* __restrict__ start) {
  __shared__ int part[kScanThreads];
  const int bh = blockIdx.x, tid = threadIdx.x;
  int32_t* hb = hist + (size_t)bh * S * C;
  int tot[2] = {0, 0};
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int c = 2 * tid + j;
    if (c < C) {
#pragma unroll 8
      for (int s = 0; s < S; ++s) tot[j] += hb[(size_t)s * C + c];
    }
  }
  const int mine = tot[0] + tot[1];
  part[tid] = mine;
  __syncthreads();
  for (int off = 1; off < kScanThreads; off <<= 1) {
    const int v = tid >= off ? part[tid - off] : 0;
    __syncthreads();
    part[tid] += v;
    __syncthreads();
  }
  int base = part[tid] - mine;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int c = 2 * tid + j;
    if (c < C) {
      start[(size_t)bh * (C + 1) + c] = base;
      int run = base;
      for (int s0 = 0; s0 < S; s0 += 8) {  // eight loads in flight before their stores
        int n[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) n[q] = s0 + q < S ? hb[(size_t)(s0 + q) * C + c] : 0;
#pragma unroll
        for (int q = 0; q < 8; ++q)
          if (s0 + q < S) {
            hb[(size_t)(s0 + q) * C + c] = run;
            run += n[q];
          }
      }
      base += tot[j];
    }
  }
  if (tid == 0) start[(size_t)bh * (C + 1) + C] = N;
}

__global__ __launch_bounds__(kWave) void order_kernel(const int32_t* __restrict__ assign,
                                                      const int32_t* __restrict__ first, int N,
                                                      int C, int S, int32_t* __restrict__ perm) {
  constexpr int PER = kSegTokens / kWave;  // tokens per lane
  __shared__ int cnt[kMaxClusters];
  const int s = blockIdx.x, bh = blockIdx.y, lane = threadIdx.x;
  const int t0 = s * kSegTokens, t1 = min(N, t0 + kSegTokens);
  // the segment's clusters, all loads in flight at once
  int ids[PER];
#pragma unroll
  for (int q = 0; q < PER; ++q) {
    const int tok = t0 + q * kWave + lane;
    ids[q] = tok < t1 ? assign[(size_t)bh * N + tok] : -1;
  }
  const int32_t* fs = first + ((size_t)bh * S + s) * C;
#pragma unroll 8
  for (int c = lane; c < C; c += kWave) cnt[c] = fs[c];
  __syncthreads();
  volatile int* vc = cnt;
  const uint64_t below = (1ull << lane) - 1ull;
#pragma unroll
  for (int q = 0; q < PER; ++q) {
    const int tok = t0 + q * kWave + lane;
    const bool ok = tok < t1;
    const int id = ids[q];
    uint64_t todo = __ballot(ok);
    int pos = 0;
    while (todo) {  // wavefront-uniform: one pass per distinct cluster among the 64 tokens
      const int leader = __ffsll((unsigned long long)todo) - 1;
      const int lid = __shfl(id, leader);
      const uint64_t peers = __ballot(id == lid);
      const int b = vc[lid];
      if (id == lid) pos = b + __popcll(peers & below);
      if (lane == leader) vc[lid] = b + __popcll(peers);
      todo &= ~peers;
    }
    if (ok) perm[(size_t)bh * N + pos] = tok;
  }
}

__global__ __launch_bounds__(256) void centroid_kernel(const __bf16* __restrict__ X,
                                                       const int32_t* __restrict__ perm,
                                                       const int32_t* __restrict__ start, int N,
                                                       int C, __bf16* __restrict__ c_hi,
                                                       __bf16* __restrict__ c_lo) {
  constexpr int D = kSvD;
  __shared__ double red[16][D];
  const int c = blockIdx.x, bh = blockIdx.y, tid = threadIdx.x;
  const int32_t* st = start + (size_t)bh * (C + 1);
  const int b0 = st[c], b1 = st[c + 1];
  if (b0 == b1) return;  // empty: the previous centroid stays (uniform over the workgroup)
  const int rg = tid / 16, col = (tid % 16) * 8;
  double acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.0;
  for (int r = b0 + rg; r < b1; r += 16) {
    const int tok = perm[(size_t)bh * N + r];
    const bf16x8 v = *reinterpret_cast<const bf16x8*>(X + ((size_t)bh * N + tok) * D + col);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] += (double)bf2f(v[e]);
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) red[rg][col + e] = acc[e];
  __syncthreads();
  if (tid < D) {
    double sum = 0.0;
#pragma unroll
    for (int r = 0; r < 16; ++r) sum += red[r][tid];
    const float m = (float)(sum / (double)(b1 - b0));
    const __bf16 hi = f2bf(m);
    c_hi[((size_t)bh * C + c) * D + tid] = hi;
    c_lo[((size_t)bh * C + c) * D + tid] = f2bf(m - bf2f(hi));
  }
}

// Rows of `words` 4-byte words; VEC4: words % 4 == 0 and 16-byte aligned rows.
template <bool VEC4>
__global__ __launch_bounds__(256) void permute_kernel(const uint32_t* __restrict__ X, int words,
                                                      const int32_t* __restrict__ perm, int N,
                                                      int scatter, uint32_t* __restrict__ Y) {
  const int bh = blockIdx.y;
  const int per = VEC4 ? words / 4 : words;  // units per row
  const size_t total = (size_t)N * per;
  const size_t hoff = (size_t)bh * N * words;
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < total; i += (size_t)gridDim.x * 256) {
    const int row = (int)(i / per), u = (int)(i % per);
    const int pr = min(max(perm[(size_t)bh * N + row], 0), N - 1);  // clamped: never outside X, Y
    const int src = scatter ? row : pr, dst = scatter ? pr : row;
    if constexpr (VEC4) {
      const i32x4 v = *reinterpret_cast<const i32x4*>(X + hoff + (size_t)src * words + 4 * u);
      *reinterpret_cast<i32x4*>(Y + hoff + (size_t)dst * words + 4 * u) = v;
    } else {
      Y[hoff + (size_t)dst * words + u] = X[hoff + (size_t)src * words + u];
    }
  }
}

}  // namespace

int svoo_segments(int N) { return (N + kSegTokens - 1) / kSegTokens; }

hipError_t launch_svoo_assign(const Dims& p, const void* X, const __bf16* c_hi,
                              const __bf16* c_lo, int32_t* assign, hipStream_t stream) {
  dim3 grid((p.N + kAssignTokens - 1) / kAssignTokens, p.B * p.H);
  assign_kernel<<<grid, kAssignThreads, 0, stream>>>((const __bf16*)X, c_hi, c_lo, p.N, p.nb,
                                                    assign);
  return hipGetLastError();
}

hipError_t launch_svoo_order(const Dims& p, const int32_t* assign, int32_t* hist, int32_t* start,
                             int32_t* perm, hipStream_t stream) {
  const int S = svoo_segments(p.N), BH = p.B * p.H;
  hist_kernel<<<dim3(S, BH), 256, 0, stream>>>(assign, p.N, p.nb, S, hist);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  scan_kernel<<<BH, kScanThreads, 0, stream>>>(hist, p.N, p.nb, S, start);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  order_kernel<<<dim3(S, BH), kWave, 0, stream>>>(assign, hist, p.N, p.nb, S, perm);
  return hipGetLastError();
}

hipError_t launch_svoo_centroids(const Dims& p, const void* X, const int32_t* perm,
                                 const int32_t* start, __bf16* c_hi, __bf16* c_lo,
                                 hipStream_t stream) {
  centroid_kernel<<<dim3(p.nb, p.B * p.H), 256, 0, stream>>>((const __bf16*)X, perm, start, p.N,
                                                            p.nb, c_hi, c_lo);
  return hipGetLastError();
}

hipError_t launch_permute_rows(const Dims& p, const void* X, int row_bytes, const int32_t* perm,
                               void* Y, int scatter, hipStream_t stream) {
  const int words = row_bytes / 4;
  const bool vec4 = row_bytes % 16 == 0 && ((uintptr_t)X % 16) == 0 && ((uintptr_t)Y % 16) == 0;
  const size_t units = (size_t)p.N * (vec4 ? words / 4 : words);
  const int gx = (int)std::min<size_t>((units + 255) / 256, 1024);
  dim3 grid(gx, p.B * p.H);
  if (vec4)
    permute_kernel<true><<<grid, 256, 0, stream>>>((const uint32_t*)X, words, perm, p.N, scatter,
                                                  (uint32_t*)Y);
  else
    permute_kernel<false><<<grid, 256, 0, stream>>>((const uint32_t*)X, words, perm, p.N, scatter,
                                                   (uint32_t*)Y);
  return hipGetLastError();
}

}  // namespace sla
